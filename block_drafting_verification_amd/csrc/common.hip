// Host-side common pieces of libdsp: error reporting, kernel timing, the
// Philox utility entry point.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "dsp_internal.h"

namespace dsp {

static thread_local char g_err[512] = {0};

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

int32_t hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSP_OK;
  return fail(DSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- timing
struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};
static int32_t g_prof_mask = 0;
static std::vector<ProfRec> g_prof_recs;
static std::vector<hipEvent_t> g_prof_pool;

static hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

bool prof_events(int kernel, hipEvent_t* start, hipEvent_t* stop) {
  if (!(g_prof_mask & (1 << kernel))) return false;
  hipEvent_t a = prof_event();
  if (!a) return false;
  hipEvent_t b = prof_event();
  if (!b) {
    g_prof_pool.push_back(a);
    return false;
  }
  *start = a;
  *stop = b;
  return true;
}

void prof_commit(int kernel, hipEvent_t start, hipEvent_t stop) { g_prof_recs.push_back({kernel, start, stop}); }

// ---------------------------------------------------------------- options
static int64_t g_options[4] = {0, 1 << 20, 1, 0};

int64_t option(int32_t opt) { return opt >= 0 && opt < 4 ? g_options[opt] : 0; }

// ---------------------------------------------------------------- philox utility
__global__ void philox_uniforms_kernel(const uint64_t* __restrict__ ctr, int64_t n, uint64_t seed,
                                       double* __restrict__ out) {
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n;
       j += (int64_t)gridDim.x * blockDim.x) {
    uint64_t c[4] = {ctr[4 * j], ctr[4 * j + 1], ctr[4 * j + 2], ctr[4 * j + 3]};
    philox4x64_10(c, seed, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w) out[4 * j + w] = unit_double(c[w]);
  }
}

}  // namespace dsp

using namespace dsp;

extern "C" int32_t dsp_version(void) { return (1 << 16) | 0; }

extern "C" const char* dsp_last_error(void) { return g_err; }

extern "C" int32_t dsp_philox_uniforms(const uint64_t* ctr, int64_t n, uint64_t seed, double* out,
                                       void* stream) {
  clear_error();
  if (n < 0) return fail(DSP_ERR_SHAPE, "n must be >= 0");
  if (n == 0) return DSP_OK;
  if (!ctr || !out) return fail(DSP_ERR_NULL, "ctr and out are required");
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  philox_uniforms_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(ctr, n, seed, out);
  return hip_check(hipGetLastError(), "philox_uniforms launch");
}

extern "C" int32_t dsp_set_option(int32_t opt, int64_t value) {
  clear_error();
  if (opt < 0 || opt >= 4) return fail(DSP_ERR_SHAPE, "unknown option %d", opt);
  if (value < 0 || (opt == DSP_OPT_SPIN_LIMIT && value > 0xffffffffll))
    return fail(DSP_ERR_SHAPE, "option %d: value out of range", opt);
  g_options[opt] = value;
  return DSP_OK;
}

extern "C" int32_t dsp_prof_enable(int32_t mask) {
  g_prof_mask = mask;
  return DSP_OK;
}

extern "C" int32_t dsp_prof_reset(void) {
  for (auto& r : g_prof_recs) {
    (void)hipEventSynchronize(r.b);
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  return DSP_OK;
}

extern "C" int32_t dsp_prof_query(int32_t kernel, double* total_ms, int64_t* launches) {
  clear_error();
  if (kernel < 0 || kernel >= DSP_K_COUNT) return fail(DSP_ERR_SHAPE, "unknown kernel id");
  if (!total_ms || !launches) return fail(DSP_ERR_NULL, "outputs required");
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_prof_recs) {
    if (r.kernel != kernel) continue;
    int32_t rc = hip_check(hipEventSynchronize(r.b), "hipEventSynchronize");
    if (rc) return rc;
    float ms = 0.f;
    rc = hip_check(hipEventElapsedTime(&ms, r.a, r.b), "hipEventElapsedTime");
    if (rc) return rc;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return DSP_OK;
}

// ---------------------------------------------------------------- read probe
namespace dsp {
namespace {
typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
// Grid-stride read of n 16-byte vectors, eight in flight per thread; the values feed a
// conditional store so the loads cannot be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4p* __restrict__ p, long n, uint32_t* sink) {
  uint32_t acc = 0;
  const long stride = (long)gridDim.x * 256;
  for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < n; v += 8 * stride) {
    u32x4p b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = v + j * stride < n ? __builtin_nontemporal_load(p + v + j * stride) : u32x4p{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= b[j].x ^ b[j].y ^ b[j].z ^ b[j].w;
  }
  // the data decide a store the compiler cannot prove dead (a single shared word would
  // serialise one atomic per wavefront)
  if (acc == 0x9E3779B9u) *sink = acc;
}
}  // namespace
}  // namespace dsp

extern "C" int32_t dsp_stream_read(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  dsp::clear_error();
  if (!p || !sink) return dsp::fail(DSP_ERR_NULL, "p and sink are required");
  if (((uintptr_t)p) % 16 || bytes % 16) return dsp::fail(DSP_ERR_ALIGN, "p and bytes must be 16-byte multiples");
  const long n = (long)(bytes / 16);
  const long want = (n + 8 * 256 - 1) / (8 * 256);
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 8192 ? 8192 : want));
  dsp::stream_read_kernel<<<dim3(grid), dim3(256), 0, (hipStream_t)stream>>>((const dsp::u32x4p*)p, n, sink);
  return dsp::hip_check(hipGetLastError(), "stream read launch");
}
