// C ABI of libkvc: argument validation (before any HIP call), workspace sizing, dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kvc.h"
#include "kvc_internal.h"

// Device workspace of kvc_correct_noalloc (see scratch_address below).
static __device__ __align__(256) unsigned char scratch[KVC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

kvc_status fail(kvc_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kvc_status ok() {
  g_err[0] = '\0';
  return KVC_OK;
}

kvc_status hip_fail(hipError_t e, const char* what) {
  return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr long long kMaxElems = 1ll << 62;

int elem_size(int dtype) { return dtype == KVC_BF16 ? 2 : 4; }

// Shape of a cache.  Returns KVC_OK or the failing status (message set).
kvc_status check_cache_shape(int L, int H, int T, int d, int dtype) {
  if (L < 0 || H < 0 || T < 0) return fail(KVC_ERR_ARG, "negative size (L=%d H=%d T=%d)", L, H, T);
  if (d <= 0) return fail(KVC_ERR_ARG, "d must be positive (d=%d)", d);
  if (dtype != KVC_BF16 && dtype != KVC_F32) return fail(KVC_ERR_ARG, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(KVC_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", d);
  const long long S = (long long)L * H;
  if (S > 65535) return fail(KVC_ERR_UNSUPPORTED, "L*H=%lld exceeds 65535 segments", S);
  if (S * T > kMaxElems / (2ll * d)) return fail(KVC_ERR_ARG, "cache too large");
  return KVC_OK;
}

kvc_status check_tensor(const void* p, const char* name, size_t align = 16) {
  if (p == nullptr) return fail(KVC_ERR_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(KVC_ERR_ARG, "%s is not %zu-byte aligned", name, align);
  return KVC_OK;
}

// Anchor shape: 1 <= A, 1 <= r <= d, A * r <= 256 (both dtypes).  Shapes outside the
// specialised kernel's budget take the general correction (kvc::correct_specialised).
kvc_status check_anchors(int A, int r, int d) {
  if (A < 1) return fail(KVC_ERR_ARG, "A=%d (need >= 1)", A);
  if (r < 1) return fail(KVC_ERR_ARG, "r=%d (need >= 1)", r);
  if (r > d) return fail(KVC_ERR_ARG, "r=%d exceeds d=%d", r, d);
  if ((long long)A * r > kvc::kMaxAnchorsGeneral)
    return fail(KVC_ERR_UNSUPPORTED, "A*r=%lld exceeds %d", (long long)A * r,
                kvc::kMaxAnchorsGeneral);
  return KVC_OK;
}

#define KVC_TRY(x)                       \
  do {                                   \
    kvc_status _s = (x);                 \
    if (_s != KVC_OK) return _s;         \
  } while (0)

#define KVC_HIP(call, what)                          \
  do {                                               \
    hipError_t _e = (call);                          \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// ---- workspace of kvc_correct_noalloc: one array per device, held until the process ends.
// In host code `scratch` names a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever handed to kernels.
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices] = {};
std::mutex g_scratch_mu;

kvc_status scratch_address(void** out) {
  int dev = -1;
  KVC_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(KVC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    KVC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(KVC_ERR_HIP, "scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace

extern "C" {

const char* kvc_version(void) { return "kvc 0.1.0 gfx950"; }

const char* kvc_last_error(void) { return g_err; }


// --------------------------------------------------------------------------- pooling
size_t kvc_pool_workspace_bytes(int L, int H, int T, int d) {
  if (L < 0 || H < 0 || T < 0 || d <= 0) return 0;
  return kvc::correct_layout(L, H, T, d, 1).off_next;  // the pooling partials only
}

kvc_status kvc_pool_descriptor(const void* K, const void* V, int L, int H, int T, int d,
                               int dtype, float* q_out, void* ws, size_t ws_bytes,
                               void* stream) {
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  const int S = L * H;
  if (S == 0) return ok();
  if (T > 0) {
    KVC_TRY(check_tensor(K, "K"));
    KVC_TRY(check_tensor(V, "V"));
  }
  KVC_TRY(check_tensor(q_out, "q_out", 4));
  const size_t need = kvc_pool_workspace_bytes(L, H, T, d);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, 1);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + c.off_pool);
  const int nc = kvc::chunks_of(T, d, dtype);
  KVC_HIP(kvc::launch_pool_partials(K, V, S, T, d, dtype, part, nc, st), "pool");
  KVC_HIP(kvc::launch_reduce_pool(part, nc, T, S, d, q_out, st), "pool reduce");
  return ok();
}

// --------------------------------------------------------------------------- correction
size_t kvc_correct_workspace_bytes(int L, int H, int T, int d, int A, int r) {
  (void)r;
  if (L < 0 || H < 0 || T < 0 || d <= 0 || A < 1) return 0;
  return kvc::correct_layout(L, H, T, d, A).bytes;
}

static kvc_status validate_correct(const void* K, const void* V, int L, int H, int T, int d,
                                   int dtype, const float* desc, const void* U, const void* W,
                                   int A, int r, const float* q_in, const void* K_fb,
                                   const void* V_fb, void* K_out, void* V_out,
                                   uint8_t* mask_out, void* ws, size_t ws_bytes) {
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  KVC_TRY(check_anchors(A, r, d));
  if (L * H == 0) return KVC_OK;
  if (T > 0) {
    KVC_TRY(check_tensor(K, "K"));
    KVC_TRY(check_tensor(V, "V"));
    KVC_TRY(check_tensor(U, "U"));
    KVC_TRY(check_tensor(K_out, "K_out"));
    KVC_TRY(check_tensor(V_out, "V_out"));
  }
  KVC_TRY(check_tensor(desc, "desc", 4));
  KVC_TRY(check_tensor(W, "W"));
  KVC_TRY(check_tensor(mask_out, "mask_out", 1));
  if (q_in != nullptr) KVC_TRY(check_tensor(q_in, "q_in", 4));
  if ((K_fb == nullptr) != (V_fb == nullptr))
    return fail(KVC_ERR_ARG, "K_fb and V_fb must both be given or both be NULL");
  if (K_fb != nullptr && T > 0) {
    KVC_TRY(check_tensor(K_fb, "K_fb"));
    KVC_TRY(check_tensor(V_fb, "V_fb"));
  }
  const size_t need = kvc_correct_workspace_bytes(L, H, T, d, A, r);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  return KVC_OK;
}

// The general correction (anchor shapes outside the specialised kernel): q from q_in, from the
// previous pass's output chunk sums, or from a pooling pass; matching of any number of
// anchors; the correction; then, if asked, the output's chunk sums by a pooling pass.
static kvc_status enqueue_correct_general(const void* K, const void* V, int L, int H, int T,
                                          int d, int dtype, const float* desc, const void* U,
                                          const void* W, int A, int r, float tau,
                                          const float* q_in, const float* next_partials_in,
                                          const void* K_fb, const void* V_fb, void* K_out,
                                          void* V_out, uint8_t* mask_out, float* score_out,
                                          float* w_out, bool want_next, void* ws,
                                          hipStream_t st) {
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
  const int nc = kvc::chunks_of(T, d, dtype);
  char* base = static_cast<char*>(ws);
  float* pool = reinterpret_cast<float*>(base + c.off_pool);
  float* qws = reinterpret_cast<float*>(base + c.off_q);
  const float* q = q_in;
  if (q == nullptr) {
    const float* part = next_partials_in;
    if (part == nullptr) {
      KVC_HIP(kvc::launch_pool_partials(K, V, c.S, T, d, dtype, pool, nc, st), "pool");
      part = pool;
    }
    KVC_HIP(kvc::launch_reduce_pool(part, nc, T, c.S, d, qws, st), "pool reduce");
    q = qws;
  }
  kvc::CorrectLaunch cl{};
  cl.K = K;
  cl.V = V;
  cl.S = c.S;
  cl.T = T;
  cl.d = d;
  cl.dtype = dtype;
  cl.U = U;
  cl.W = W;
  cl.A = A;
  cl.r = r;
  cl.w_ws = reinterpret_cast<float*>(base + c.off_w);
  cl.mask_ws = reinterpret_cast<uint8_t*>(base + c.off_mask);
  cl.K_fb = K_fb;
  cl.V_fb = V_fb;
  cl.K_out = K_out;
  cl.V_out = V_out;
  KVC_HIP(kvc::launch_score_general(q, desc, c.S, d, A, tau, cl.w_ws,
                                    reinterpret_cast<uint8_t*>(base + c.off_mask), score_out,
                                    w_out, mask_out, st),
          "score");
  KVC_HIP(kvc::launch_correct_general(cl, st), "correct");
  if (want_next)
    KVC_HIP(kvc::launch_pool_partials(K_out, V_out, c.S, T, d, dtype,
                                      reinterpret_cast<float*>(base + c.off_next), nc, st),
            "pool of the output");
  return KVC_OK;
}

// One correction pass: the pooled descriptor from q_in, from the chunk sums that the previous
// pass of a chain left in the workspace, or from a pooling pass over (K, V); then the matching
// kernel (cosines, softmax, score, flag) and the correction kernel, whose output chunk sums
// serve the next pass when asked.
static kvc_status enqueue_correct(const void* K, const void* V, int L, int H, int T, int d,
                                  int dtype, const float* desc, const void* U, const void* W,
                                  int A, int r, float tau, const float* q_in,
                                  const float* next_partials_in, const void* K_fb,
                                  const void* V_fb, void* K_out, void* V_out,
                                  uint8_t* mask_out, float* score_out, float* w_out,
                                  bool want_next, void* ws, hipStream_t st) {
  if (!kvc::correct_specialised(A, r, dtype))
    return enqueue_correct_general(K, V, L, H, T, d, dtype, desc, U, W, A, r, tau, q_in,
                                   next_partials_in, K_fb, V_fb, K_out, V_out, mask_out,
                                   score_out, w_out, want_next, ws, st);
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
  const int nc = kvc::chunks_of(T, d, dtype);
  char* base = static_cast<char*>(ws);
  float* pool = reinterpret_cast<float*>(base + c.off_pool);
  kvc::CorrectLaunch cl{};
  cl.K = K;
  cl.V = V;
  cl.S = c.S;
  cl.T = T;
  cl.d = d;
  cl.dtype = dtype;
  cl.U = U;
  cl.W = W;
  cl.A = A;
  cl.r = r;
  cl.w_ws = reinterpret_cast<float*>(base + c.off_w);
  cl.mask_ws = reinterpret_cast<uint8_t*>(base + c.off_mask);
  cl.K_fb = K_fb;
  cl.V_fb = V_fb;
  cl.K_out = K_out;
  cl.V_out = V_out;
  cl.next_partials = want_next ? reinterpret_cast<float*>(base + c.off_next) : nullptr;
  cl.ctr = reinterpret_cast<int*>(base + c.off_ctr);
  const float* part = next_partials_in;
  if (q_in == nullptr && part == nullptr) {
    KVC_HIP(kvc::launch_pool_partials(K, V, c.S, T, d, dtype, pool, nc, st), "pool");
    part = pool;
  }
  KVC_HIP(kvc::launch_score(part, nc, T, q_in, desc, c.S, d, A, tau, cl.w_ws,
                            reinterpret_cast<uint8_t*>(base + c.off_mask), score_out, w_out,
                            mask_out, cl.ctr, st),
          "score");
  KVC_HIP(kvc::launch_correct(cl, st), "correct");
  return KVC_OK;
}

kvc_status kvc_correct(const void* K, const void* V, int L, int H, int T, int d, int dtype,
                       const float* desc, const void* U, const void* W, int A, int r,
                       float tau, const float* q_in, const void* K_fb, const void* V_fb,
                       void* K_out, void* V_out, uint8_t* mask_out, float* score_out,
                       float* w_out, float* q_next_out, void* ws, size_t ws_bytes,
                       void* stream) {
  KVC_TRY(validate_correct(K, V, L, H, T, d, dtype, desc, U, W, A, r, q_in, K_fb, V_fb, K_out,
                           V_out, mask_out, ws, ws_bytes));
  if (score_out) KVC_TRY(check_tensor(score_out, "score_out", 4));
  if (w_out) KVC_TRY(check_tensor(w_out, "w_out", 4));
  if (q_next_out) KVC_TRY(check_tensor(q_next_out, "q_next_out", 4));
  if (L * H == 0) return ok();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  KVC_TRY(enqueue_correct(K, V, L, H, T, d, dtype, desc, U, W, A, r, tau, q_in, nullptr, K_fb,
                          V_fb, K_out, V_out, mask_out, score_out, w_out, q_next_out != nullptr,
                          ws, st));
  if (q_next_out) {
    const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
    float* next = reinterpret_cast<float*>(static_cast<char*>(ws) + c.off_next);
    KVC_HIP(kvc::launch_reduce_pool(next, kvc::chunks_of(T, d, dtype), T, c.S, d, q_next_out, st),
            "q_next");
  }
  return ok();
}

kvc_status kvc_correct_noalloc(const void* K, const void* V, int L, int H, int T, int d,
                               int dtype, const float* desc, const void* U, const void* W, int A,
                               int r, float tau, const float* q_in, const void* K_fb,
                               const void* V_fb, void* K_out, void* V_out, uint8_t* mask_out,
                               float* score_out, float* w_out, float* q_next_out,
                               void* stream) {
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  KVC_TRY(check_anchors(A, r, d));
  const size_t need = kvc_correct_workspace_bytes(L, H, T, d, A, r);
  if (need > (size_t)KVC_SCRATCH_BYTES)
    return fail(KVC_ERR_UNSUPPORTED,
                "needs %zu bytes of workspace, more than the %u-byte scratch array", need,
                (unsigned)KVC_SCRATCH_BYTES);
  void* ws = nullptr;
  KVC_TRY(scratch_address(&ws));
  return kvc_correct(K, V, L, H, T, d, dtype, desc, U, W, A, r, tau, q_in, K_fb, V_fb, K_out,
                     V_out, mask_out, score_out, w_out, q_next_out, ws, KVC_SCRATCH_BYTES,
                     stream);
}

// --------------------------------------------------------------------------- chain
size_t kvc_chain_workspace_bytes(int L, int H, int T, int d, int A, int r) {
  return kvc_correct_workspace_bytes(L, H, T, d, A, r);
}

kvc_status kvc_correct_chain(const void* K0, const void* V0, int L, int H, int T, int d,
                             int dtype, int n_edges, const float* const* desc,
                             const void* const* U, const void* const* W, int A, int r,
                             float tau, const void* const* K_fb, const void* const* V_fb,
                             void* const* K_out, void* const* V_out,
                             uint8_t* const* mask_out, float* const* score_out, void* ws,
                             size_t ws_bytes, void* stream) {
  if (n_edges < 1) return fail(KVC_ERR_ARG, "n_edges=%d (need >= 1)", n_edges);
  if (!desc || !U || !W || !K_out || !V_out || !mask_out)
    return fail(KVC_ERR_ARG, "desc, U, W, K_out, V_out and mask_out arrays are required");
  if ((K_fb == nullptr) != (V_fb == nullptr))
    return fail(KVC_ERR_ARG, "K_fb and V_fb arrays must both be given or both be NULL");
  for (int e = 0; e < n_edges; ++e) {
    const void* src_k = e == 0 ? K0 : K_out[e - 1];
    const void* src_v = e == 0 ? V0 : V_out[e - 1];
    const void* kf = K_fb ? K_fb[e] : nullptr;
    const void* vf = V_fb ? V_fb[e] : nullptr;
    kvc_status s = validate_correct(src_k, src_v, L, H, T, d, dtype, desc[e], U[e], W[e], A, r,
                                    nullptr, kf, vf, K_out[e], V_out[e], mask_out[e], ws,
                                    ws_bytes);
    if (s != KVC_OK) {
      char tmp[512];
      snprintf(tmp, sizeof(tmp), "edge %d: %s", e, g_err);
      return fail(s, "%s", tmp);
    }
    if (score_out && score_out[e]) KVC_TRY(check_tensor(score_out[e], "score_out[e]", 4));
    if (T > 0 && (K_out[e] == src_k || V_out[e] == src_v))
      return fail(KVC_ERR_ARG, "edge %d writes over its own source", e);
  }
  if (L * H == 0) return ok();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
  const float* next = reinterpret_cast<const float*>(static_cast<char*>(ws) + c.off_next);
  for (int e = 0; e < n_edges; ++e) {
    const void* src_k = e == 0 ? K0 : K_out[e - 1];
    const void* src_v = e == 0 ? V0 : V_out[e - 1];
    const void* kf = K_fb ? K_fb[e] : nullptr;
    const void* vf = V_fb ? V_fb[e] : nullptr;
    KVC_TRY(enqueue_correct(src_k, src_v, L, H, T, d, dtype, desc[e], U[e], W[e], A, r, tau,
                            nullptr, e == 0 ? nullptr : next, kf, vf, K_out[e], V_out[e],
                            mask_out[e], score_out ? score_out[e] : nullptr, nullptr,
                            e + 1 < n_edges, ws, st));
  }
  return ok();
}

// --------------------------------------------------------------------------- fanout
size_t kvc_fanout_workspace_bytes(int L, int H, int T, int d, int A, int r) {
  return kvc_correct_workspace_bytes(L, H, T, d, A, r);
}

static bool overlaps(const void* a, const void* b, size_t n) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + n && y < x + n;
}

kvc_status kvc_correct_fanout(const void* K, const void* V, int L, int H, int T, int d,
                              int dtype, int n_agents, const float* const* desc,
                              const void* const* U, const void* const* W, int A, int r,
                              float tau, const void* const* K_fb, const void* const* V_fb,
                              void* const* K_out, void* const* V_out,
                              uint8_t* const* mask_out, float* const* score_out, void* ws,
                              size_t ws_bytes, void* stream) {
  if (n_agents < 1) return fail(KVC_ERR_ARG, "n_agents=%d (need >= 1)", n_agents);
  if (!desc || !U || !W || !K_out || !V_out || !mask_out)
    return fail(KVC_ERR_ARG, "desc, U, W, K_out, V_out and mask_out arrays are required");
  if ((K_fb == nullptr) != (V_fb == nullptr))
    return fail(KVC_ERR_ARG, "K_fb and V_fb arrays must both be given or both be NULL");
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  const size_t cache_bytes = (size_t)L * H * T * d * elem_size(dtype);
  for (int j = 0; j < n_agents; ++j) {
    const void* kf = K_fb ? K_fb[j] : nullptr;
    const void* vf = V_fb ? V_fb[j] : nullptr;
    kvc_status s = validate_correct(K, V, L, H, T, d, dtype, desc[j], U[j], W[j], A, r, nullptr,
                                    kf, vf, K_out[j], V_out[j], mask_out[j], ws, ws_bytes);
    if (s != KVC_OK) {
      char tmp[512];
      snprintf(tmp, sizeof(tmp), "agent %d: %s", j, g_err);
      return fail(s, "%s", tmp);
    }
    if (score_out && score_out[j]) KVC_TRY(check_tensor(score_out[j], "score_out[j]", 4));
    if (cache_bytes == 0) continue;
    const void* outs[2] = {K_out[j], V_out[j]};
    for (const void* o : outs) {
      if (overlaps(o, K, cache_bytes) || overlaps(o, V, cache_bytes))
        return fail(KVC_ERR_ARG, "agent %d writes over the shared reference cache", j);
      for (int i = 0; i < j; ++i)
        if (overlaps(o, K_out[i], cache_bytes) || overlaps(o, V_out[i], cache_bytes))
          return fail(KVC_ERR_ARG, "outputs of agents %d and %d overlap", i, j);
    }
    if (overlaps(K_out[j], V_out[j], cache_bytes))
      return fail(KVC_ERR_ARG, "agent %d: K_out and V_out overlap", j);
  }
  if (L * H == 0) return ok();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n_agents == 1) {  // one agent: exactly kvc_correct
    KVC_TRY(enqueue_correct(K, V, L, H, T, d, dtype, desc[0], U[0], W[0], A, r, tau, nullptr,
                            nullptr, K_fb ? K_fb[0] : nullptr, V_fb ? V_fb[0] : nullptr,
                            K_out[0], V_out[0], mask_out[0], score_out ? score_out[0] : nullptr,
                            nullptr, false, ws, st));
    return ok();
  }
  // Several agents: the reference is pooled once; each agent is matched from those chunk sums
  // (the same pooled descriptor, bit for bit); then one launch per group of up to kMaxTargets
  // agents reads each tile of the reference once and corrects it for every agent of the group.
  // Anchor shapes outside the specialised kernel: the general correction, agent by agent, all
  // matched against the reference's one pooled descriptor.
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
  const int nc = kvc::chunks_of(T, d, dtype);
  char* base = static_cast<char*>(ws);
  float* pool = reinterpret_cast<float*>(base + c.off_pool);
  if (!kvc::correct_specialised(A, r, dtype)) {
    float* qws = reinterpret_cast<float*>(base + c.off_q);
    KVC_HIP(kvc::launch_pool_partials(K, V, c.S, T, d, dtype, pool, nc, st), "pool");
    KVC_HIP(kvc::launch_reduce_pool(pool, nc, T, c.S, d, qws, st), "pool reduce");
    for (int j = 0; j < n_agents; ++j)
      KVC_TRY(enqueue_correct_general(K, V, L, H, T, d, dtype, desc[j], U[j], W[j], A, r, tau,
                                      qws, nullptr, K_fb ? K_fb[j] : nullptr,
                                      V_fb ? V_fb[j] : nullptr, K_out[j], V_out[j],
                                      mask_out[j], score_out ? score_out[j] : nullptr, nullptr,
                                      false, ws, st));
    return ok();
  }
  float* wmt = reinterpret_cast<float*>(base + c.off_wmt);
  uint8_t* mmt = reinterpret_cast<uint8_t*>(base + c.off_mmt);
  int* ctr = reinterpret_cast<int*>(base + c.off_ctr);
  KVC_HIP(kvc::launch_pool_partials(K, V, c.S, T, d, dtype, pool, nc, st), "pool");
  for (int j0 = 0; j0 < n_agents; j0 += kvc::kMaxTargets) {
    const int n = n_agents - j0 < kvc::kMaxTargets ? n_agents - j0 : kvc::kMaxTargets;
    kvc::CorrectLaunch cl{};
    cl.K = K;
    cl.V = V;
    cl.S = c.S;
    cl.T = T;
    cl.d = d;
    cl.dtype = dtype;
    cl.U = U[j0];
    cl.W = W[j0];
    cl.A = A;
    cl.r = r;
    cl.w_ws = wmt;
    cl.mask_ws = mmt;
    cl.K_out = K_out[j0];
    cl.V_out = V_out[j0];
    cl.ctr = ctr;
    cl.n_t = n;
    for (int j = 0; j < n; ++j) {
      const int g = j0 + j;
      KVC_HIP(kvc::launch_score(pool, nc, T, nullptr, desc[g], c.S, d, A, tau,
                                wmt + (size_t)j * c.S * A, mmt + (size_t)j * c.S,
                                score_out ? score_out[g] : nullptr, nullptr, mask_out[g], ctr,
                                st),
              "score");
      cl.tU[j] = U[g];
      cl.tW[j] = W[g];
      cl.tK[j] = K_out[g];
      cl.tV[j] = V_out[g];
      cl.tKfb[j] = K_fb ? K_fb[g] : nullptr;
      cl.tVfb[j] = V_fb ? V_fb[g] : nullptr;
    }
    KVC_HIP(kvc::launch_correct(cl, st), "correct");
  }
  return ok();
}

// --------------------------------------------------------------------------- rank matching
size_t kvc_rank_descriptor_workspace_bytes(int L, int H, int T, int d, int rC) {
  if (L < 0 || H < 0 || T < 0 || d <= 0 || rC < 1) return 0;
  const int S = L * H;
  const size_t fit = kvc::fit_layout(2 * S, T, d, rC).bytes;
  const size_t eig = kvc::align_up(sizeof(float) * 2ull * S * d, 256);
  const size_t ke = kvc::align_up(sizeof(int32_t) * 2ull * S, 256);
  return fit + eig + ke;
}

kvc_status kvc_rank_descriptor(const void* K, const void* V, int L, int H, int T, int d,
                               int dtype, int rC, float* F_out, int32_t* k_eff_out, void* ws,
                               size_t ws_bytes, void* stream) {
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  if (rC < 1 || rC > d || rC > kvc::kMaxRankC)
    return fail(KVC_ERR_ARG, "rC=%d (need 1 <= rC <= d)", rC);
  const int S = L * H;
  if (S == 0) return ok();
  if (T > 0) {
    KVC_TRY(check_tensor(K, "K"));
    KVC_TRY(check_tensor(V, "V"));
  }
  KVC_TRY(check_tensor(F_out, "F_out"));
  if (k_eff_out) KVC_TRY(check_tensor(k_eff_out, "k_eff_out", 4));
  const size_t need = kvc_rank_descriptor_workspace_bytes(L, H, T, d, rC);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  char* base = static_cast<char*>(ws);
  const size_t fit = kvc::fit_layout(2 * S, T, d, rC).bytes;
  float* eig = reinterpret_cast<float*>(base + fit);
  int32_t* ke = k_eff_out ? k_eff_out
                          : reinterpret_cast<int32_t*>(
                                base + fit + kvc::align_up(sizeof(float) * 2ull * S * d, 256));
  KVC_HIP(kvc::launch_rank_descriptor(K, V, S, T, d, dtype, rC, F_out, ke, eig, base,
                                      reinterpret_cast<hipStream_t>(stream)),
          "rank descriptor");
  return ok();
}

kvc_status kvc_correct_rank(const void* K, const void* V, int L, int H, int T, int d, int dtype,
                            const float* Fq, const float* Fa, int rC, const void* U,
                            const void* W, int A, int r, float tau, const void* K_fb,
                            const void* V_fb, void* K_out, void* V_out, uint8_t* mask_out,
                            float* score_out, float* w_out, void* ws, size_t ws_bytes,
                            void* stream) {
  if (L > 0 && H > 0) KVC_TRY(check_tensor(Fq, "Fq", 4));
  KVC_TRY(validate_correct(K, V, L, H, T, d, dtype, Fq, U, W, A, r, nullptr, K_fb, V_fb, K_out,
                           V_out, mask_out, ws, ws_bytes));
  if (rC < 1 || rC > d || rC > kvc::kMaxRankC)
    return fail(KVC_ERR_ARG, "rC=%d (need 1 <= rC <= d)", rC);
  if (score_out) KVC_TRY(check_tensor(score_out, "score_out", 4));
  if (w_out) KVC_TRY(check_tensor(w_out, "w_out", 4));
  if (L * H == 0) return ok();
  KVC_TRY(check_tensor(Fa, "Fa", 4));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
  char* base = static_cast<char*>(ws);
  kvc::CorrectLaunch cl{};
  cl.K = K;
  cl.V = V;
  cl.S = c.S;
  cl.T = T;
  cl.d = d;
  cl.dtype = dtype;
  cl.U = U;
  cl.W = W;
  cl.A = A;
  cl.r = r;
  cl.w_ws = reinterpret_cast<float*>(base + c.off_w);
  cl.mask_ws = reinterpret_cast<uint8_t*>(base + c.off_mask);
  cl.K_fb = K_fb;
  cl.V_fb = V_fb;
  cl.K_out = K_out;
  cl.V_out = V_out;
  cl.ctr = reinterpret_cast<int*>(base + c.off_ctr);
  KVC_HIP(kvc::launch_score_rank(Fq, Fa, c.S, d, A, rC, tau, cl.w_ws,
                                 reinterpret_cast<uint8_t*>(base + c.off_mask), score_out, w_out,
                                 mask_out, cl.ctr, st),
          "rank matching");
  if (kvc::correct_specialised(A, r, dtype))
    KVC_HIP(kvc::launch_correct(cl, st), "correct");
  else
    KVC_HIP(kvc::launch_correct_general(cl, st), "correct");
  return ok();
}

// --------------------------------------------------------------------------- anchor pool
size_t kvc_correct_pooled_workspace_bytes(int L, int H, int T, int d, int A, int r) {
  return kvc_correct_workspace_bytes(L, H, T, d, A, r);
}

static kvc_status check_pool(int Vc, int A) {
  if (Vc < 1) return fail(KVC_ERR_ARG, "Vc=%d (need >= 1)", Vc);
  if (Vc > kvc::kMaxPool)
    return fail(KVC_ERR_UNSUPPORTED, "Vc=%d exceeds %d pool slots", Vc, kvc::kMaxPool);
  if (A > Vc) return fail(KVC_ERR_ARG, "A=%d exceeds the pool capacity Vc=%d", A, Vc);
  return KVC_OK;
}

kvc_status kvc_correct_pooled(const void* K, const void* V, int L, int H, int T, int d,
                              int dtype, const float* desc_pool, const void* U_pool,
                              const void* W_pool, const int32_t* count, int Vc, int A, int r,
                              float tau, const float* q_in, const void* K_fb, const void* V_fb,
                              void* K_out, void* V_out, uint8_t* mask_out, float* score_out,
                              float* w_out, int32_t* slot_out, void* ws, size_t ws_bytes,
                              void* stream) {
  KVC_TRY(validate_correct(K, V, L, H, T, d, dtype, desc_pool, U_pool, W_pool, A, r, q_in,
                           K_fb, V_fb, K_out, V_out, mask_out, ws, ws_bytes));
  KVC_TRY(check_pool(Vc, A));
  if (score_out) KVC_TRY(check_tensor(score_out, "score_out", 4));
  if (w_out) KVC_TRY(check_tensor(w_out, "w_out", 4));
  if (slot_out) KVC_TRY(check_tensor(slot_out, "slot_out", 4));
  if (L * H == 0) return ok();
  KVC_TRY(check_tensor(count, "count", 4));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const kvc::CorrectLayout c = kvc::correct_layout(L, H, T, d, A);
  const int nc = kvc::chunks_of(T, d, dtype);
  char* base = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(base + c.off_pool);
  if (q_in == nullptr)
    KVC_HIP(kvc::launch_pool_partials(K, V, c.S, T, d, dtype, part, nc, st), "pool");
  kvc::CorrectLaunch cl{};
  cl.K = K;
  cl.V = V;
  cl.S = c.S;
  cl.T = T;
  cl.d = d;
  cl.dtype = dtype;
  cl.U = U_pool;
  cl.W = W_pool;
  cl.A = A;
  cl.r = r;
  cl.w_ws = reinterpret_cast<float*>(base + c.off_w);
  cl.mask_ws = reinterpret_cast<uint8_t*>(base + c.off_mask);
  cl.K_fb = K_fb;
  cl.V_fb = V_fb;
  cl.K_out = K_out;
  cl.V_out = V_out;
  cl.ctr = reinterpret_cast<int*>(base + c.off_ctr);
  cl.slot_ws = reinterpret_cast<int*>(base + c.off_slot);
  cl.Vc = Vc;
  KVC_HIP(kvc::launch_select(part, nc, T, q_in, desc_pool, count, Vc, c.S, d, A, tau, cl.w_ws,
                             reinterpret_cast<int*>(base + c.off_slot),
                             reinterpret_cast<uint8_t*>(base + c.off_mask), score_out, w_out,
                             slot_out, mask_out, cl.ctr, st),
          "select");
  if (kvc::correct_specialised(A, r, dtype))
    KVC_HIP(kvc::launch_correct(cl, st), "correct");
  else
    KVC_HIP(kvc::launch_correct_general(cl, st), "correct");
  return ok();
}

kvc_status kvc_anchor_pool_insert(const uint8_t* mask, const float* U_new, const float* W_new,
                                  const float* q, int L, int H, int T, int d, int dtype, int Vc,
                                  int r, void* U_pool, void* W_pool, float* desc_pool,
                                  int32_t* count, int32_t* head, void* stream) {
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  if (Vc < 1) return fail(KVC_ERR_ARG, "Vc=%d (need >= 1)", Vc);
  if (Vc > kvc::kMaxPool)
    return fail(KVC_ERR_UNSUPPORTED, "Vc=%d exceeds %d pool slots", Vc, kvc::kMaxPool);
  if (r < 1 || r > d) return fail(KVC_ERR_ARG, "r=%d (need 1 <= r <= d)", r);
  if (L * H == 0) return ok();
  KVC_TRY(check_tensor(mask, "mask", 1));
  KVC_TRY(check_tensor(W_new, "W_new", 4));
  KVC_TRY(check_tensor(q, "q", 4));
  KVC_TRY(check_tensor(W_pool, "W_pool", 4));
  KVC_TRY(check_tensor(desc_pool, "desc_pool", 4));
  KVC_TRY(check_tensor(count, "count", 4));
  KVC_TRY(check_tensor(head, "head", 4));
  if (T > 0) {
    KVC_TRY(check_tensor(U_new, "U_new", 4));
    KVC_TRY(check_tensor(U_pool, "U_pool", 4));
  }
  KVC_HIP(kvc::launch_pool_insert(mask, U_new, W_new, q, L * H, T, d, dtype, Vc, r, U_pool,
                                  W_pool, desc_pool, count, head,
                                  reinterpret_cast<hipStream_t>(stream)),
          "pool insert");
  return ok();
}

// --------------------------------------------------------------------------- error measures
size_t kvc_segment_error_workspace_bytes(int L, int H, int T, int d) {
  (void)d;
  if (L < 0 || H < 0 || T < 0) return 0;
  const size_t n = 2ull * L * H * kvc::segment_error_chunks(T) * sizeof(double);
  return n > 0 ? n : 256;
}

kvc_status kvc_segment_error(const void* X, const void* ref, int L, int H, int T, int d,
                             int dtype, double* out, void* ws, size_t ws_bytes, void* stream) {
  KVC_TRY(check_cache_shape(L, H, T, d, dtype));
  if (L * H == 0) return ok();
  if (T > 0) {
    KVC_TRY(check_tensor(X, "X"));
    KVC_TRY(check_tensor(ref, "ref"));
  }
  KVC_TRY(check_tensor(out, "out", 8));
  const size_t need = kvc_segment_error_workspace_bytes(L, H, T, d);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  KVC_HIP(kvc::launch_segment_error(X, ref, L * H, T, d, dtype, static_cast<double*>(ws), out,
                                    reinterpret_cast<hipStream_t>(stream)),
          "segment_error");
  return ok();
}

kvc_status kvc_rank_error_curve(const float* eig, int M, int n, float* curve_out, void* stream) {
  if (M < 0 || n < 1) return fail(KVC_ERR_ARG, "M=%d n=%d (need M >= 0, n >= 1)", M, n);
  if (n > kvc::rank_error_curve_max_n())
    return fail(KVC_ERR_UNSUPPORTED, "n=%d exceeds %d eigenvalues", n,
                kvc::rank_error_curve_max_n());
  if (M == 0) return ok();
  KVC_TRY(check_tensor(eig, "eig", 4));
  KVC_TRY(check_tensor(curve_out, "curve_out", 4));
  KVC_HIP(kvc::launch_rank_error_curve(eig, M, n, curve_out,
                                       reinterpret_cast<hipStream_t>(stream)),
          "rank_error_curve");
  return ok();
}

// --------------------------------------------------------------------------- fit
size_t kvc_fit_workspace_bytes(int M, int T, int d, int r) {
  if (M < 0 || T < 0 || d <= 0 || r < 1) return 0;
  return kvc::fit_layout(M, T, d, r).bytes;
}

kvc_status kvc_fit_anchor(const void* delta, int M, int T, int d, int dtype, int r,
                          double energy, float* U_out, float* W_out, int32_t* k_eff_out,
                          float* eig_out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || T < 0) return fail(KVC_ERR_ARG, "negative size (M=%d T=%d)", M, T);
  if (d <= 0) return fail(KVC_ERR_ARG, "d must be positive (d=%d)", d);
  if (dtype != KVC_BF16 && dtype != KVC_F32) return fail(KVC_ERR_ARG, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(KVC_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", d);
  if (r < 1 || r > d) return fail(KVC_ERR_ARG, "r=%d (need 1 <= r <= d)", r);
  if (!(energy > 0.0 && energy <= 1.0)) return fail(KVC_ERR_ARG, "energy must be in (0, 1]");
  if (M > 65535) return fail(KVC_ERR_UNSUPPORTED, "M=%d exceeds 65535 matrices", M);
  if ((long long)M * T > kMaxElems / (2ll * d)) return fail(KVC_ERR_ARG, "delta too large");
  if (M == 0) return ok();
  if (T > 0) {
    KVC_TRY(check_tensor(delta, "delta"));
    KVC_TRY(check_tensor(U_out, "U_out"));
  }
  KVC_TRY(check_tensor(W_out, "W_out"));
  KVC_TRY(check_tensor(k_eff_out, "k_eff_out", 4));
  if (eig_out) KVC_TRY(check_tensor(eig_out, "eig_out", 4));
  const size_t need = kvc_fit_workspace_bytes(M, T, d, r);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  const kvc::FitLayout f = kvc::fit_layout(M, T, d, r);
  KVC_HIP(kvc::launch_fit(delta, f, dtype, energy, U_out, W_out, k_eff_out, eig_out,
                          static_cast<char*>(ws), reinterpret_cast<hipStream_t>(stream)),
          "fit");
  return ok();
}

// --------------------------------------------------------------------------- streaming fit
static kvc_status validate_fit_shape(int M, int d, int dtype) {
  if (M < 0) return fail(KVC_ERR_ARG, "negative size (M=%d)", M);
  if (d <= 0) return fail(KVC_ERR_ARG, "d must be positive (d=%d)", d);
  if (dtype != KVC_BF16 && dtype != KVC_F32) return fail(KVC_ERR_ARG, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(KVC_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", d);
  if (M > 65535) return fail(KVC_ERR_UNSUPPORTED, "M=%d exceeds 65535 matrices", M);
  return KVC_OK;
}

size_t kvc_gram_workspace_bytes(int M, int T, int d) {
  if (M < 0 || T < 0 || d <= 0) return 0;
  return kvc::gram_ws_bytes(kvc::fit_layout(M, T, d, 1));
}

kvc_status kvc_gram_accumulate(const void* delta, int M, int T, int d, int dtype,
                               double* G_inout, void* ws, size_t ws_bytes, void* stream) {
  KVC_TRY(validate_fit_shape(M, d, dtype));
  if (T < 0) return fail(KVC_ERR_ARG, "negative size (T=%d)", T);
  if ((long long)M * T > kMaxElems / (2ll * d)) return fail(KVC_ERR_ARG, "delta too large");
  if (M == 0 || T == 0) return ok();
  KVC_TRY(check_tensor(delta, "delta"));
  KVC_TRY(check_tensor(G_inout, "G", 8));
  const size_t need = kvc_gram_workspace_bytes(M, T, d);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  const kvc::FitLayout f = kvc::fit_layout(M, T, d, 1);
  KVC_HIP(kvc::launch_gram_accumulate(delta, f, dtype, G_inout, static_cast<char*>(ws),
                                      reinterpret_cast<hipStream_t>(stream)),
          "gram_accumulate");
  return ok();
}

kvc_status kvc_fit_from_gram(const double* G, int M, int d, int r, double energy, float* W_out,
                             int32_t* k_eff_out, float* eig_out, void* stream) {
  KVC_TRY(validate_fit_shape(M, d, KVC_F32));
  if (r < 1 || r > d) return fail(KVC_ERR_ARG, "r=%d (need 1 <= r <= d)", r);
  if (!(energy > 0.0 && energy <= 1.0)) return fail(KVC_ERR_ARG, "energy must be in (0, 1]");
  if (M == 0) return ok();
  KVC_TRY(check_tensor(G, "G", 8));
  KVC_TRY(check_tensor(W_out, "W_out"));
  KVC_TRY(check_tensor(k_eff_out, "k_eff_out", 4));
  if (eig_out) KVC_TRY(check_tensor(eig_out, "eig_out", 4));
  KVC_HIP(kvc::launch_fit_from_gram(G, M, d, r, energy, W_out, k_eff_out, eig_out,
                                    reinterpret_cast<hipStream_t>(stream)),
          "fit_from_gram");
  return ok();
}

kvc_status kvc_refit_warm(const double* G, int M, int d, int r, double energy,
                          const float* W_prev, float* W_out, int32_t* k_eff_out,
                          int32_t* warm_out, void* stream) {
  KVC_TRY(validate_fit_shape(M, d, KVC_F32));
  if (r < 1 || r > d) return fail(KVC_ERR_ARG, "r=%d (need 1 <= r <= d)", r);
  if (!(energy > 0.0 && energy <= 1.0)) return fail(KVC_ERR_ARG, "energy must be in (0, 1]");
  if (M == 0) return ok();
  KVC_TRY(check_tensor(G, "G", 8));
  KVC_TRY(check_tensor(W_prev, "W_prev"));
  KVC_TRY(check_tensor(W_out, "W_out"));
  KVC_TRY(check_tensor(k_eff_out, "k_eff_out", 4));
  if (warm_out) KVC_TRY(check_tensor(warm_out, "warm_out", 4));
  KVC_HIP(kvc::launch_refit_warm(G, M, d, r, energy, W_prev, W_out, k_eff_out, warm_out,
                                 reinterpret_cast<hipStream_t>(stream)),
          "refit_warm");
  return ok();
}

size_t kvc_project_workspace_bytes(int M, int d, int r, int dtype) {
  if (M < 0 || d <= 0 || r < 1) return 0;
  return kvc::project_ws_bytes(M, d, r, dtype);
}

kvc_status kvc_project(const void* delta, int M, int T, int d, int dtype, const float* W, int r,
                       float* U_out, void* ws, size_t ws_bytes, void* stream) {
  KVC_TRY(validate_fit_shape(M, d, dtype));
  if (T < 0) return fail(KVC_ERR_ARG, "negative size (T=%d)", T);
  if (r < 1 || r > d) return fail(KVC_ERR_ARG, "r=%d (need 1 <= r <= d)", r);
  if ((long long)M * T > kMaxElems / (2ll * d)) return fail(KVC_ERR_ARG, "delta too large");
  if (M == 0 || T == 0) return ok();
  KVC_TRY(check_tensor(delta, "delta"));
  KVC_TRY(check_tensor(W, "W"));
  KVC_TRY(check_tensor(U_out, "U_out"));
  const size_t need = kvc_project_workspace_bytes(M, d, r, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 256)))
    return fail(KVC_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  KVC_HIP(kvc::launch_project(delta, M, T, d, dtype, W, r, U_out, static_cast<char*>(ws),
                              reinterpret_cast<hipStream_t>(stream)),
          "project");
  return ok();
}

}  // extern "C"
