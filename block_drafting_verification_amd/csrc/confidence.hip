// Confidence head with sequential temperature scaling for gfx950.
//
// Operation (DSpark study notes, section 5.1 "Confidence Head"; SGLang article,
// Sequential Temperature Scaling): for every draft position k of request i,
// c_{i,k} = sigmoid((w . h_{i,k} + b) / T_k), the probability that the draft
// survives verification given that the earlier ones did; T_k calibrates the
// position (1 when no temperatures are given). The scheduler multiplies these
// into block survival probabilities.
//
// One wavefront per (i, k) row, four rows per 256-thread workgroup: the row's H
// hidden values stream in as 16-byte vectors, each lane forms fp32 partial dot
// products per vector with the weights (read once per workgroup from L2) and adds
// them in fp64; a butterfly sums the lanes; the logit, the temperature and the
// sigmoid are fp64. The pass is HBM-bound: R*K*H element reads.
#include <math.h>

#include "dsp_internal.h"

namespace dsp {
namespace {

constexpr int kConfRows = 4;  // rows (wavefronts) per workgroup
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {  // bf16: one 16-byte vector holds 8 values
  static constexpr int kVecs = 1;
  __device__ static void unpack(const u32x4* w, float* x) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = bf16_lo(w[0][q]);
      x[2 * q + 1] = bf16_hi(w[0][q]);
    }
  }
  __device__ static float val(const uint16_t* p, long j) { return bf16_val(p[j]); }
};
template <> struct Vec8<float> {  // fp32: two vectors
  static constexpr int kVecs = 2;
  __device__ static void unpack(const u32x4* w, float* x) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = __uint_as_float(w[0][q]);
      x[4 + q] = __uint_as_float(w[1][q]);
    }
  }
  __device__ static float val(const float* p, long j) { return p[j]; }
};

struct ConfArgs {
  const void* h;
  int64_t ld_r, ld_k;
  const void* w;
  float bias;
  const float* temps;
  int32_t R, K, H;
  float* conf;
  int32_t* status;
};

template <typename TH, typename TW>
__global__ __launch_bounds__(64 * kConfRows) void confidence_kernel(ConfArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kConfRows + (threadIdx.x >> 6);
  if (row >= (long)a.R * a.K) return;  // uniform over the wavefront
  const int i = (int)(row / a.K), k = (int)(row % a.K);
  const TH* hp = (const TH*)a.h + (size_t)i * a.ld_r + (size_t)k * a.ld_k;
  const TW* wp = (const TW*)a.w;
  // 8-element groups; the vector path needs both rows 16-byte aligned
  const bool al = ((((uintptr_t)hp) | ((uintptr_t)wp)) & 15u) == 0;
  const int ng = a.H / 8;
  double acc = 0.0;
  int g = lane;
  if (al) {
    constexpr int B = 8;  // groups per lane in flight (a whole 4096-wide bf16 row per wavefront)
    for (; g + 64 * (B - 1) < ng; g += 64 * B) {
      u32x4 hv[B][Vec8<TH>::kVecs], wv[B][Vec8<TW>::kVecs];
#pragma unroll
      for (int b = 0; b < B; ++b) {
#pragma unroll
        for (int q = 0; q < Vec8<TH>::kVecs; ++q)
          hv[b][q] = __builtin_nontemporal_load((const u32x4*)(hp + 8 * (g + 64 * b)) + q);
#pragma unroll
        for (int q = 0; q < Vec8<TW>::kVecs; ++q) wv[b][q] = *((const u32x4*)(wp + 8 * (g + 64 * b)) + q);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float x[8], y[8];
        Vec8<TH>::unpack(hv[b], x);
        Vec8<TW>::unpack(wv[b], y);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf(x[e], y[e], s);
        acc += (double)s;
      }
    }
  }
  for (; g < ng; g += 64) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf(Vec8<TH>::val(hp, 8 * g + e), Vec8<TW>::val(wp, 8 * g + e), s);
    acc += (double)s;
  }
  if (lane < a.H - 8 * ng) acc += (double)Vec8<TH>::val(hp, 8 * ng + lane) * (double)Vec8<TW>::val(wp, 8 * ng + lane);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) {
    double logit = acc + (double)a.bias;
    if (a.temps) logit /= (double)a.temps[k];
    const double c = 1.0 / (1.0 + exp(-logit));
    a.conf[row] = (float)c;
    if (!(c == c)) atomicOr(a.status, DSP_STATUS_NONFINITE);
  }
}

}  // namespace
}  // namespace dsp

using namespace dsp;

extern "C" int32_t dsp_confidence_head(const void* h, int32_t h_dtype, int64_t ld_h_r, int64_t ld_h_k,
                                       const void* w, int32_t w_dtype, float bias, const float* sts_temp,
                                       int32_t R, int32_t K, int32_t H, float* conf, int32_t* status,
                                       void* stream) {
  clear_error();
  if (R < 1 || K < 1 || H < 1) return fail(DSP_ERR_SHAPE, "need R, K, H >= 1 (R=%d K=%d H=%d)", R, K, H);
  if ((h_dtype != DSP_F32 && h_dtype != DSP_BF16) || (w_dtype != DSP_F32 && w_dtype != DSP_BF16))
    return fail(DSP_ERR_DTYPE, "hidden states and weights must be f32 or bf16");
  if (!h || !w || !conf || !status) return fail(DSP_ERR_NULL, "h, w, conf and status are required");
  if (ld_h_k < H || ld_h_r < (int64_t)(K - 1) * ld_h_k + H) return fail(DSP_ERR_SHAPE, "h strides too small");
  const size_t eh = h_dtype == DSP_BF16 ? 2 : 4, ew = w_dtype == DSP_BF16 ? 2 : 4;
  if (((uintptr_t)h) % eh || ((uintptr_t)w) % ew) return fail(DSP_ERR_ALIGN, "h and w must be element aligned");
  ConfArgs a{h, ld_h_r, ld_h_k, w, bias, sts_temp, R, K, H, conf, status};
  const long rows = (long)R * K;
  const dim3 grid((unsigned)((rows + kConfRows - 1) / kConfRows)), block(64 * kConfRows);
  hipStream_t s = (hipStream_t)stream;
  if (h_dtype == DSP_BF16 && w_dtype == DSP_BF16) launch(DSP_K_CONFIDENCE, confidence_kernel<uint16_t, uint16_t>, grid, block, 0, s, a);
  else if (h_dtype == DSP_BF16) launch(DSP_K_CONFIDENCE, confidence_kernel<uint16_t, float>, grid, block, 0, s, a);
  else if (w_dtype == DSP_BF16) launch(DSP_K_CONFIDENCE, confidence_kernel<float, uint16_t>, grid, block, 0, s, a);
  else launch(DSP_K_CONFIDENCE, confidence_kernel<float, float>, grid, block, 0, s, a);
  return hip_check(hipGetLastError(), "confidence head launch");
}
