// C ABI of the library: argument validation, workspace carve-up and launches on the
// caller's stream.  Validation mirrors the host launchers on the pages (boostr
// flash_bwd.rs: shape, contiguity and dtype checks returning InvalidArgument before any
// launch; rustytorch backward.rs: shape checks and "not on the device" errors), adapted to
// raw pointers: shapes arrive as integers, so what is checked here is what pointers and
// sizes can express; the Python binding checks tensor shapes, strides and devices.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/fab.h"
#include "launch.h"

// Static scratch of fab_bwd_noalloc, for callers that cannot allocate device memory: it holds
// the per-row statistics {lse * log2(e), D} that fab_bwd keeps in its workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device copy: host code uses only the address that
// hipGetSymbolAddress returns for the current device (scratch_device_ptr below).
constexpr size_t kScratchBytes = size_t(16) << 20;  // 2^21 padded query rows of 8 bytes
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

fab_status fail(fab_status s, const char* arg, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(arg) + ": " + buf;
  return s;
}

bool log_enabled() {
  static int v = [] {
    const char* e = getenv("FAB_LOG");
    return (e && e[0] && e[0] != '0') ? 1 : 0;
  }();
  return v != 0;
}

void log_launch(const fab::LaunchInfo& li) {
  if (log_enabled())
    fprintf(stderr, "[fab] %s grid=%d block=%d lds=%d B\n", li.name, li.grid, li.block, li.lds_bytes);
}

#define FAB_TRY(x)                    \
  do {                                \
    fab_status s_ = (x);              \
    if (s_ != FAB_OK) return s_;      \
  } while (0)

constexpr long long kMaxElems = (1LL << 31) - 1;

size_t elem_size(int dt) { return dt == FAB_F32 ? 4 : 2; }

// Which kernels run: bf16 / fp16 take the tiled kernels (fwd16.hip, bwd16.hip) at every head
// dim; fp32 takes the generic ones (fwd.hip, bwd_dkdv.hip, bwd_dq.hip).
bool tiled(int dtype) { return dtype != FAB_F32; }

fab_status check_common(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype) {
  if (dtype != FAB_F32 && dtype != FAB_F16 && dtype != FAB_BF16)
    return fail(FAB_ERR_UNSUPPORTED, "dtype", "unsupported dtype code %d (expected 0=f32, 1=f16, 2=bf16)", dtype);
  if (B < 1 || H < 1 || H_kv < 1 || Sq < 1 || Sk < 1 || D < 1)
    return fail(FAB_ERR_INVALID_ARGUMENT, "dims",
                "every size must be >= 1 (B=%d H=%d H_kv=%d Sq=%d Sk=%d D=%d)", B, H, H_kv, Sq, Sk, D);
  if (D != 32 && D != 64 && D != 96 && D != 128 && !(D == 256 && dtype != FAB_F32))
    return fail(FAB_ERR_UNSUPPORTED, "head_dim",
                "head dim %d not supported (32, 64, 96, 128; also 256 for f16/bf16)", D);
  if (H % H_kv != 0)
    return fail(FAB_ERR_INVALID_ARGUMENT, "num_kv_heads",
                "num_heads %d is not a multiple of num_kv_heads %d", H, H_kv);
  if ((long long)B * H * Sq * D > kMaxElems || (long long)B * H_kv * Sk * D > kMaxElems)
    return fail(FAB_ERR_INVALID_ARGUMENT, "dims", "a tensor exceeds 2^31-1 elements");
  // The kernels address the row statistics of one kv-head group with 32-bit byte offsets.
  if ((long long)(H / H_kv) * fab::stats_rows(Sq) * 8 > 0xFFFFFFFFLL)
    return fail(FAB_ERR_UNSUPPORTED, "dims",
                "num_heads / num_kv_heads * Sq too large (%d query heads per kv head, Sq=%d)", H / H_kv, Sq);
  return FAB_OK;
}

fab_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FAB_ERR_INVALID_ARGUMENT, name, "null pointer");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(FAB_ERR_INVALID_ARGUMENT, name, "pointer %p is not 16-byte aligned", p);
  return FAB_OK;
}

// The pointer must be device memory of the current device whose allocation covers
// [p, p + bytes).  Run after the cheap checks, so invalid arguments never touch the runtime.
fab_status check_device_range(const void* p, size_t bytes, const char* name) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(FAB_ERR_DEVICE, name, "no usable GPU (%s)", hipGetErrorString(e));
  hipPointerAttribute_t attr;
  e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess || attr.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return fail(FAB_ERR_DEVICE, name, "pointer %p is not device memory", p);
  }
  if (attr.device != dev)
    return fail(FAB_ERR_DEVICE, name, "pointer is on device %d, current device is %d", attr.device, dev);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FAB_ERR_DEVICE, name, "cannot query the allocation of %p", p);
  }
  const char* lo = static_cast<const char*>(base);
  const char* q = static_cast<const char*>(p);
  if (q < lo || (size_t)(q - lo) + bytes > size)
    return fail(FAB_ERR_DEVICE, name, "allocation holds %zu bytes from %p, tensor needs %zu",
                size - (size_t)(q - lo), p, bytes);
  return FAB_OK;
}

// Workspace: the per-row statistics, B * H * Sq_pad float pairs, rounded up to 256 bytes.
size_t ws_bytes(long long B, long long H, long long Sq) {
  const size_t d = (size_t)(B * H) * fab::stats_rows((int)Sq) * 8;
  return (d + 255) / 256 * 256;
}

// Stored-dS mode (16-bit inputs): the workspace also holds every dS fragment the dK/dV kernel
// forms, one slab of ds_rows(Sq) x ds_keys(Sk) 16-bit values per (b, h), from a 4 KB
// boundary after the statistics.  The kernels address a slab with 32-bit offsets (a group's G
// slabs with one buffer resource), and the whole buffer is capped so that the mode stays a
// choice for sizes where memory is plentiful; beyond, dQ recomputes dS.
constexpr unsigned long long kDsMaxBytes = 32ULL << 30;

unsigned long long ds_slab_bytes(int Sq, int Sk) {
  return (unsigned long long)fab::ds_rows(Sq) * (unsigned long long)fab::ds_keys(Sk) * 2ULL;
}

bool ds_mode_fits(int B, int H, int H_kv, int Sq, int Sk, int dtype) {
  if (dtype == FAB_F32) return false;
  const unsigned long long slab = ds_slab_bytes(Sq, Sk);
  return slab <= (1ULL << 31) && (unsigned long long)(H / H_kv) * slab < (1ULL << 32) &&
         (unsigned long long)B * H * slab <= kDsMaxBytes;
}

size_t ds_offset(int B, int H, int Sq) { return (ws_bytes(B, H, Sq) + 4095) / 4096 * 4096; }

size_t ws_bytes_ds(int B, int H, int Sq, int Sk) {
  return ds_offset(B, H, Sq) + (size_t)B * H * ds_slab_bytes(Sq, Sk);
}

// The workspace selects the mode: with at least ws_bytes_ds (and sizes the mode takes) the
// dK/dV kernel stores dS and dQ reads it back; with less (at least ws_bytes) dQ recomputes it.
bool use_ds(size_t given, int B, int H, int H_kv, int Sq, int Sk, int dtype) {
  return ds_mode_fits(B, H, H_kv, Sq, Sk, dtype) && given >= ws_bytes_ds(B, H, Sq, Sk);
}

int units_per_xcd(int n_units) { return n_units % 8 == 0 ? n_units / 8 : 0; }

fab_status check_window(int window_size) {
  if (window_size < 0)
    return fail(FAB_ERR_INVALID_ARGUMENT, "window_size", "%d is negative (0 = no window)", window_size);
  return FAB_OK;
}

// The window as the kernels take it: 0 for none, and also for a window of at least
// max(Sq, Sk) keys, which cuts no (query, key) pair of these sizes.
int kernel_window(int window_size, int Sq, int Sk) {
  return window_size >= (Sq > Sk ? Sq : Sk) ? 0 : window_size;
}

fab::BwdParams bwd_params(const void* dO, const void* q, const void* k, const void* v,
                          const void* workspace, void* dq, void* dk, void* dv,
                          int B, int H, int H_kv, int Sq, int Sk, int causal, int window_size,
                          float scale) {
  fab::BwdParams p;
  p.q = q; p.k = k; p.v = v; p.dO = dO; p.stats = static_cast<const float*>(workspace);
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.o = nullptr; p.lse = nullptr; p.stats_out = nullptr;
  p.ds = nullptr; p.ds_slab = 0; p.ds_nk32 = 0;
  p.B = B; p.H = H; p.H_kv = H_kv; p.Sq = Sq; p.Sk = Sk; p.Sq_pad = fab::stats_rows(Sq);
  p.causal = causal ? 1 : 0;
  p.win = kernel_window(window_size, Sq, Sk);
  p.scale = scale;
  // The kernels mask a score by replacing it with mask_s, for which mask_s * scale_log2 is
  // -inf.  A zero (or subnormal) exponent scale is raised to the smallest normal float of the
  // same sign so that this product is never 0 * inf; the scores it multiplies are finite, and
  // s * FLT_MIN is far below the resolution of the exponent's other term.
  float sl2 = scale * fab::kLog2eHost;
  if (std::fabs(sl2) < FLT_MIN) sl2 = std::signbit(sl2) ? -FLT_MIN : FLT_MIN;
  p.scale_log2 = sl2;
  p.mask_s = sl2 > 0.f ? -INFINITY : INFINITY;
  p.n_units = B * H_kv;
  p.units_per_xcd = units_per_xcd(p.n_units);
  return p;
}

// The dK/dV kernel writes the dS region, the dQ kernel only reads it.
void set_ds(fab::BwdParams& p, const void* workspace) {
  p.ds = const_cast<char*>(static_cast<const char*>(workspace)) + ds_offset(p.B, p.H, p.Sq);
  p.ds_slab = (unsigned)ds_slab_bytes(p.Sq, p.Sk);
  p.ds_nk32 = (int)(fab::ds_keys(p.Sk) / 32);
}

// The mode fab_bwd_workspace_bytes recommends: stored dS where it applies, measured faster
// from head dim 96 up (it moves 2 bytes of dS per allowed pair to save 4 D FLOPs of recompute,
// which below D = 96 cost less than the traffic), and not for problems small enough for the
// single fused launch of the recomputing kernels.
bool recommend_ds(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype) {
  if (D < 96 || !ds_mode_fits(B, H, H_kv, Sq, Sk, dtype)) return false;
  const fab::BwdParams p =
      bwd_params(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 B, H, H_kv, Sq, Sk, 0, 0, 1.f);
  return !fab::bwd_small16_fits(p, D);
}

// Checks shared by fab_bwd and the two step-2 entry points (every pointer but dq/dk/dv).
fab_status check_bwd_inputs(const void* dO, const void* q, const void* k, const void* v,
                            int B, int H, int H_kv, int Sq, int Sk, int D, int dtype,
                            int window_size, float scale) {
  FAB_TRY(check_common(B, H, H_kv, Sq, Sk, D, dtype));
  FAB_TRY(check_window(window_size));
  FAB_TRY(check_ptr(dO, "dO"));
  FAB_TRY(check_ptr(q, "q"));
  FAB_TRY(check_ptr(k, "k"));
  FAB_TRY(check_ptr(v, "v"));
  if (!std::isfinite(scale)) return fail(FAB_ERR_INVALID_ARGUMENT, "scale", "scale must be finite");
  return FAB_OK;
}

fab_status check_bwd_device(const void* dO, const void* q, const void* k, const void* v,
                            int B, int H, int H_kv, int Sq, int Sk, int D, int dtype) {
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H * Sq * D * es, nk = (size_t)B * H_kv * Sk * D * es;
  FAB_TRY(check_device_range(dO, nq, "dO"));
  FAB_TRY(check_device_range(q, nq, "q"));
  FAB_TRY(check_device_range(k, nk, "k"));
  FAB_TRY(check_device_range(v, nk, "v"));
  return FAB_OK;
}

fab_status check_workspace(const void* ws, size_t given, int B, int H, int Sq) {
  FAB_TRY(check_ptr(ws, "workspace"));
  const size_t need = ws_bytes(B, H, Sq);
  if (given < need)
    return fail(FAB_ERR_INVALID_ARGUMENT, "workspace", "%zu bytes given, %zu needed", given, need);
  return FAB_OK;
}

fab::PreParams pre_params(const void* dO, const void* o, const float* lse, void* ws, int B, int H, int Sq) {
  fab::PreParams pp;
  pp.dO = dO; pp.o = o; pp.lse = lse; pp.stats = static_cast<float*>(ws);
  pp.BH = B * H; pp.Sq = Sq; pp.Sq_pad = fab::stats_rows(Sq);
  return pp;
}

hipError_t launch_step2(const fab::BwdParams& p, int dtype, int D, hipStream_t s, bool dkdv, bool dq,
                        fab::LaunchInfo* li) {
  hipError_t e = hipSuccess;
  if (dkdv) {
    e = tiled(dtype) ? fab::launch_bwd_dkdv16(p, dtype, D, s, li) : fab::launch_bwd_dkdv(p, dtype, D, s, li);
    if (e != hipSuccess) return e;
    log_launch(*li);
  }
  if (dq) {
    e = tiled(dtype) ? fab::launch_bwd_dq16(p, dtype, D, s, li) : fab::launch_bwd_dq(p, dtype, D, s, li);
    if (e != hipSuccess) return e;
    log_launch(*li);
  }
  return e;
}

fab_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FAB_ERR_LAUNCH, what, "launch failed: %s", hipGetErrorString(e));
  return FAB_OK;
}

// Device address of the current device's copy of `scratch`, looked up once per device (with
// that device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fab_status scratch_device_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FAB_ERR_DEVICE, "scratch", "no usable GPU (%s)", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FAB_ERR_DEVICE, "scratch", "device index %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return fail(FAB_ERR_DEVICE, "scratch", "hipGetSymbolAddress failed on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FAB_OK;
}

// The launches of the backward, after validation.  `workspace` holds the per-row statistics.
fab_status run_bwd(const void* dO, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace, bool ds,
                   int B, int H, int H_kv, int Sq, int Sk, int D, int dtype, int causal,
                   int window_size, float scale, hipStream_t s) {
  fab::LaunchInfo li;
  fab::BwdParams p =
      bwd_params(dO, q, k, v, workspace, dq, dk, dv, B, H, H_kv, Sq, Sk, causal, window_size, scale);
  if (ds) {
    // Stored dS: step 1, then the dK/dV kernel (which also writes dS), then dQ = scale dS K.
    set_ds(p, workspace);
    const fab::PreParams pp = pre_params(dO, o, lse, workspace, B, H, Sq);
    FAB_TRY(launched(fab::launch_preprocess(pp, dtype, D, s, &li), "preprocess"));
    log_launch(li);
    FAB_TRY(launched(launch_step2(p, dtype, D, s, true, false, &li), "bwd_dkdv"));
    FAB_TRY(launched(fab::launch_bwd_dq_ds16(p, dtype, D, s, &li), "bwd_dq"));
    log_launch(li);
    return FAB_OK;
  }
  if (tiled(dtype) && fab::bwd_small16_fits(p, D)) {
    // A small problem: step 1, then both step-2 kernels in one launch, which fills the device
    // where each grid alone would leave it half idle.
    const fab::PreParams pp = pre_params(dO, o, lse, workspace, B, H, Sq);
    FAB_TRY(launched(fab::launch_preprocess(pp, dtype, D, s, &li), "preprocess"));
    log_launch(li);
    FAB_TRY(launched(fab::launch_bwd_small16(p, dtype, D, s, &li), "bwd_small"));
    log_launch(li);
    return FAB_OK;
  }
  if (tiled(dtype)) {
    // Step 1 runs inside the dQ kernel, which therefore goes first: it writes the row
    // statistics the dK/dV kernel then reads from the workspace.
    fab::BwdParams pq = p;
    pq.o = o; pq.lse = lse; pq.stats_out = static_cast<float*>(workspace);
    FAB_TRY(launched(fab::launch_bwd_dq16(pq, dtype, D, s, &li), "bwd_dq"));
    log_launch(li);
    FAB_TRY(launched(launch_step2(p, dtype, D, s, true, false, &li), "bwd_dkdv"));
    return FAB_OK;
  }
  const fab::PreParams pp = pre_params(dO, o, lse, workspace, B, H, Sq);
  FAB_TRY(launched(fab::launch_preprocess(pp, dtype, D, s, &li), "preprocess"));
  log_launch(li);
  FAB_TRY(launched(launch_step2(p, dtype, D, s, true, true, &li), "step 2"));
  return FAB_OK;
}

}  // namespace

extern "C" {

const char* fab_version(void) { return "fab 0.1.0 (gfx950)"; }

const char* fab_last_error(void) { return g_last_error.c_str(); }

size_t fab_bwd_workspace_bytes(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype) {
  std::string saved = g_last_error;
  fab_status s = check_common(B, H, H_kv, Sq, Sk, D, dtype);
  g_last_error = saved;
  if (s != FAB_OK) return 0;
  return recommend_ds(B, H, H_kv, Sq, Sk, D, dtype) ? ws_bytes_ds(B, H, Sq, Sk) : ws_bytes(B, H, Sq);
}

int fab_bwd_plan(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype, size_t workspace_bytes) {
  std::string saved = g_last_error;
  fab_status s = check_common(B, H, H_kv, Sq, Sk, D, dtype);
  g_last_error = saved;
  if (s != FAB_OK || workspace_bytes < ws_bytes(B, H, Sq)) return -1;
  if (!tiled(dtype)) return FAB_PLAN_F32;
  if (use_ds(workspace_bytes, B, H, H_kv, Sq, Sk, dtype)) return FAB_PLAN_STORED_DS;
  const fab::BwdParams p =
      bwd_params(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 B, H, H_kv, Sq, Sk, 0, 0, 1.f);
  return fab::bwd_small16_fits(p, D) ? FAB_PLAN_RECOMPUTE_ONE_LAUNCH : FAB_PLAN_RECOMPUTE;
}

size_t fab_bwd_workspace_bytes_ds(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype) {
  std::string saved = g_last_error;
  fab_status s = check_common(B, H, H_kv, Sq, Sk, D, dtype);
  g_last_error = saved;
  if (s != FAB_OK || !ds_mode_fits(B, H, H_kv, Sq, Sk, dtype)) return 0;
  return ws_bytes_ds(B, H, Sq, Sk);
}

size_t fab_bwd_workspace_bytes_min(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype) {
  std::string saved = g_last_error;
  fab_status s = check_common(B, H, H_kv, Sq, Sk, D, dtype);
  g_last_error = saved;
  if (s != FAB_OK) return 0;
  return ws_bytes(B, H, Sq);
}

fab_status fab_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int Sq, int Sk, int D, int dtype,
                   int causal, int window_size, float scale, void* stream) {
  FAB_TRY(check_common(B, H, H_kv, Sq, Sk, D, dtype));
  FAB_TRY(check_window(window_size));
  FAB_TRY(check_ptr(q, "q"));
  FAB_TRY(check_ptr(k, "k"));
  FAB_TRY(check_ptr(v, "v"));
  FAB_TRY(check_ptr(o, "o"));
  FAB_TRY(check_ptr(lse, "lse"));
  if (!std::isfinite(scale)) return fail(FAB_ERR_INVALID_ARGUMENT, "scale", "scale must be finite");
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H * Sq * D * es, nk = (size_t)B * H_kv * Sk * D * es;
  FAB_TRY(check_device_range(q, nq, "q"));
  FAB_TRY(check_device_range(k, nk, "k"));
  FAB_TRY(check_device_range(v, nk, "v"));
  FAB_TRY(check_device_range(o, nq, "o"));
  FAB_TRY(check_device_range(lse, (size_t)B * H * Sq * 4, "lse"));

  fab::FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.H_kv = H_kv; p.Sq = Sq; p.Sk = Sk;
  p.causal = causal ? 1 : 0;
  p.win = kernel_window(window_size, Sq, Sk);
  p.scale = scale;
  p.scale_log2 = scale * fab::kLog2eHost;
  p.n_units = B * H_kv;
  p.units_per_xcd = units_per_xcd(p.n_units);
  fab::LaunchInfo li;
  const hipError_t e = tiled(dtype) ? fab::launch_fwd16(p, dtype, D, (hipStream_t)stream, &li)
                                       : fab::launch_fwd(p, dtype, D, (hipStream_t)stream, &li);
  FAB_TRY(launched(e, "fwd"));
  log_launch(li);
  return FAB_OK;
}

fab_status fab_bwd_preprocess(const void* dO, const void* o, const float* lse,
                              void* workspace, size_t workspace_bytes,
                              int B, int H, int Sq, int D, int dtype, void* stream) {
  FAB_TRY(check_common(B, H, H, Sq, 1, D, dtype));
  FAB_TRY(check_ptr(dO, "dO"));
  FAB_TRY(check_ptr(o, "o"));
  FAB_TRY(check_ptr(lse, "lse"));
  FAB_TRY(check_workspace(workspace, workspace_bytes, B, H, Sq));
  const size_t nq = (size_t)B * H * Sq * D * elem_size(dtype);
  FAB_TRY(check_device_range(dO, nq, "dO"));
  FAB_TRY(check_device_range(o, nq, "o"));
  FAB_TRY(check_device_range(lse, (size_t)B * H * Sq * 4, "lse"));
  FAB_TRY(check_device_range(workspace, ws_bytes(B, H, Sq), "workspace"));
  const fab::PreParams pp = pre_params(dO, o, lse, workspace, B, H, Sq);
  fab::LaunchInfo li;
  FAB_TRY(launched(fab::launch_preprocess(pp, dtype, D, (hipStream_t)stream, &li), "preprocess"));
  log_launch(li);
  return FAB_OK;
}

fab_status fab_bwd(const void* dO, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int H_kv, int Sq, int Sk, int D, int dtype,
                   int causal, int window_size, float scale, void* stream) {
  FAB_TRY(check_bwd_inputs(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype, window_size, scale));
  FAB_TRY(check_ptr(o, "o"));
  FAB_TRY(check_ptr(lse, "lse"));
  FAB_TRY(check_ptr(dq, "dq"));
  FAB_TRY(check_ptr(dk, "dk"));
  FAB_TRY(check_ptr(dv, "dv"));
  FAB_TRY(check_workspace(workspace, workspace_bytes, B, H, Sq));
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H * Sq * D * es, nk = (size_t)B * H_kv * Sk * D * es;
  FAB_TRY(check_bwd_device(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype));
  FAB_TRY(check_device_range(o, nq, "o"));
  FAB_TRY(check_device_range(lse, (size_t)B * H * Sq * 4, "lse"));
  FAB_TRY(check_device_range(dq, nq, "dq"));
  FAB_TRY(check_device_range(dk, nk, "dk"));
  FAB_TRY(check_device_range(dv, nk, "dv"));
  const bool ds = use_ds(workspace_bytes, B, H, H_kv, Sq, Sk, dtype);
  FAB_TRY(check_device_range(workspace, ds ? ws_bytes_ds(B, H, Sq, Sk) : ws_bytes(B, H, Sq), "workspace"));

  return run_bwd(dO, q, k, v, o, lse, dq, dk, dv, workspace, ds, B, H, H_kv, Sq, Sk, D, dtype,
                 causal, window_size, scale, (hipStream_t)stream);
}

fab_status fab_bwd_noalloc(const void* dO, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, void* dq, void* dk, void* dv,
                           int B, int H, int H_kv, int Sq, int Sk, int D, int dtype,
                           int causal, int window_size, float scale, void* stream) {
  FAB_TRY(check_bwd_inputs(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype, window_size, scale));
  FAB_TRY(check_ptr(o, "o"));
  FAB_TRY(check_ptr(lse, "lse"));
  FAB_TRY(check_ptr(dq, "dq"));
  FAB_TRY(check_ptr(dk, "dk"));
  FAB_TRY(check_ptr(dv, "dv"));
  const size_t need = ws_bytes(B, H, Sq);
  if (need > kScratchBytes)
    return fail(FAB_ERR_INVALID_ARGUMENT, "dims",
                "needs %zu bytes of statistics (B * num_heads * Sq rounded up to 64 = %lld rows), "
                "the static scratch holds %zu (%zu rows)", need,
                (long long)B * H * fab::stats_rows(Sq), kScratchBytes, kScratchBytes / 8);
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H * Sq * D * es, nk = (size_t)B * H_kv * Sk * D * es;
  FAB_TRY(check_bwd_device(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype));
  FAB_TRY(check_device_range(o, nq, "o"));
  FAB_TRY(check_device_range(lse, (size_t)B * H * Sq * 4, "lse"));
  FAB_TRY(check_device_range(dq, nq, "dq"));
  FAB_TRY(check_device_range(dk, nk, "dk"));
  FAB_TRY(check_device_range(dv, nk, "dv"));
  void* ws = nullptr;
  FAB_TRY(scratch_device_ptr(&ws));
  return run_bwd(dO, q, k, v, o, lse, dq, dk, dv, ws, false, B, H, H_kv, Sq, Sk, D, dtype, causal,
                 window_size, scale, (hipStream_t)stream);
}

fab_status fab_bwd_dkdv(const void* dO, const void* q, const void* k, const void* v,
                        void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int H, int H_kv, int Sq, int Sk, int D,
                        int dtype, int causal, int window_size, float scale, void* stream) {
  FAB_TRY(check_bwd_inputs(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype, window_size, scale));
  FAB_TRY(check_ptr(dk, "dk"));
  FAB_TRY(check_ptr(dv, "dv"));
  FAB_TRY(check_workspace(workspace, workspace_bytes, B, H, Sq));
  const size_t nk = (size_t)B * H_kv * Sk * D * elem_size(dtype);
  FAB_TRY(check_bwd_device(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype));
  const bool ds = use_ds(workspace_bytes, B, H, H_kv, Sq, Sk, dtype);
  FAB_TRY(check_device_range(workspace, ds ? ws_bytes_ds(B, H, Sq, Sk) : ws_bytes(B, H, Sq), "workspace"));
  FAB_TRY(check_device_range(dk, nk, "dk"));
  FAB_TRY(check_device_range(dv, nk, "dv"));
  fab::BwdParams p =
      bwd_params(dO, q, k, v, workspace, nullptr, dk, dv, B, H, H_kv, Sq, Sk, causal, window_size, scale);
  if (ds) set_ds(p, workspace);
  fab::LaunchInfo li;
  FAB_TRY(launched(launch_step2(p, dtype, D, (hipStream_t)stream, true, false, &li), "bwd_dkdv"));
  return FAB_OK;
}

fab_status fab_bwd_dq(const void* dO, const void* q, const void* k, const void* v,
                      const void* workspace, size_t workspace_bytes, void* dq,
                      int B, int H, int H_kv, int Sq, int Sk, int D,
                      int dtype, int causal, int window_size, float scale, void* stream) {
  FAB_TRY(check_bwd_inputs(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype, window_size, scale));
  FAB_TRY(check_ptr(dq, "dq"));
  FAB_TRY(check_workspace(workspace, workspace_bytes, B, H, Sq));
  const size_t nq = (size_t)B * H * Sq * D * elem_size(dtype);
  FAB_TRY(check_bwd_device(dO, q, k, v, B, H, H_kv, Sq, Sk, D, dtype));
  const bool ds = use_ds(workspace_bytes, B, H, H_kv, Sq, Sk, dtype);
  FAB_TRY(check_device_range(workspace, ds ? ws_bytes_ds(B, H, Sq, Sk) : ws_bytes(B, H, Sq), "workspace"));
  FAB_TRY(check_device_range(dq, nq, "dq"));
  fab::BwdParams p =
      bwd_params(dO, q, k, v, workspace, dq, nullptr, nullptr, B, H, H_kv, Sq, Sk, causal, window_size, scale);
  fab::LaunchInfo li;
  if (ds) {
    set_ds(p, workspace);
    FAB_TRY(launched(fab::launch_bwd_dq_ds16(p, dtype, D, (hipStream_t)stream, &li), "bwd_dq"));
    log_launch(li);
    return FAB_OK;
  }
  FAB_TRY(launched(launch_step2(p, dtype, D, (hipStream_t)stream, false, true, &li), "bwd_dq"));
  return FAB_OK;
}

}  // extern "C"
