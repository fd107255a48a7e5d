// Calibration of the confidences against the verify's outcomes for gfx950.
//
// Operation (SGLang article, observability: per-request confidences and calibration
// metrics such as ECE beside the acceptance ceiling; DSpark study notes, section 5.1:
// c_{i,k} is the probability that draft position k survives given every earlier
// position was accepted). With window n_i = cu[i+1] - cu[i] - 1 and m_i drafts accepted
// over the decided window (the accepted length, or the cap-accept ceiling), positions
// k = 1..m_i have outcome 1 and position m_i + 1 <= n_i outcome 0; later positions were
// never decided. Binned expected calibration error with B equal-width bins of [0, 1]
// (bin floor(c * B) in fp64, clamped to [0, B-1]):
//   ECE = (1/n) * sum_b | sum over bin b of (outcome - c) |,
// which equals sum_b (n_b / n) |mean outcome_b - mean c_b|; 0 when nothing was observed.
//
// One workgroup of 1024 threads: each wavefront takes requests in turn, one draft
// position per lane (K <= 64), and reduces per bin with fixed butterflies; the batch's
// per-bin sums are kept per wavefront and combined in a fixed order, so the results are
// deterministic bit for bit.
#include <math.h>

#include "dsp_internal.h"

namespace dsp {
namespace {

constexpr int kCalThreads = 1024;
constexpr int kCalWaves = kCalThreads / 64;
constexpr int kMaxBins = 64;

struct CalArgs {
  const float* conf;
  int64_t ld_conf;
  const int32_t* cu;
  const int32_t* decided;
  int32_t R, K, B;
  double* ece;
  int32_t* n_obs;
  double* batch;  // [1 + 3B]: batch ECE, per-bin count, sum of c, sum of outcomes
};

__device__ __forceinline__ double wsum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(kCalThreads) void calibration_kernel(CalArgs a) {
  __shared__ double s_cnt[kCalWaves][kMaxBins], s_c[kCalWaves][kMaxBins], s_o[kCalWaves][kMaxBins];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // lane b keeps this wavefront's batch sums of bin b
  double bc = 0.0, bsc = 0.0, bso = 0.0;
  for (int i = w; i < a.R; i += kCalWaves) {
    const int n = a.cu[i + 1] - a.cu[i] - 1;
    const int m = a.decided[i];
    const int last = (m < 0 || n <= 0 || n > a.K) ? 0 : min(n, m + 1);
    const bool obs = lane < last;
    const double c = obs ? (double)a.conf[(size_t)i * a.ld_conf + lane] : 0.0;
    const double o = lane < m ? 1.0 : 0.0;
    const double bf = floor(c * (double)a.B);  // exact for fp32 c; NaN lands in bin 0
    const int b = bf >= (double)a.B ? a.B - 1 : (bf > 0.0 ? (int)bf : 0);
    double e = 0.0;
    for (int j = 0; j < a.B; ++j) {  // uniform: every lane takes part in every reduction
      const bool in = obs && b == j;
      const double d = wsum(in ? o - c : 0.0);
      const double sc = wsum(in ? c : 0.0), so = wsum(in ? o : 0.0);
      const double cnt = (double)__popcll(__ballot(in));
      e += fabs(d);
      if (lane == j) {  // lane b keeps the batch sums of bin b
        bc += cnt;
        bsc += sc;
        bso += so;
      }
    }
    if (lane == 0) {
      a.ece[i] = last > 0 ? e / (double)last : 0.0;
      a.n_obs[i] = last;
    }
  }
  if (lane < kMaxBins) {
    s_cnt[w][lane] = bc;
    s_c[w][lane] = bsc;
    s_o[w][lane] = bso;
  }
  __syncthreads();
  if (w == 0) {
    double cnt = 0.0, sc = 0.0, so = 0.0;
    for (int q = 0; q < kCalWaves; ++q) {
      cnt += s_cnt[q][lane];
      sc += s_c[q][lane];
      so += s_o[q][lane];
    }
    const bool live = lane < a.B;
    const double n = wsum(live ? cnt : 0.0);
    const double e = wsum(live ? fabs(so - sc) : 0.0);
    if (live) {
      a.batch[1 + lane] = cnt;
      a.batch[1 + a.B + lane] = sc;
      a.batch[1 + 2 * a.B + lane] = so;
    }
    if (lane == 0) a.batch[0] = n > 0.0 ? e / n : 0.0;
  }
}

}  // namespace
}  // namespace dsp

using namespace dsp;

extern "C" int32_t dsp_verify_calibration(const float* conf, int64_t ld_conf, const int32_t* cu_seqlens,
                                          const int32_t* decided, int32_t R, int32_t K, int32_t n_bins,
                                          double* ece, int32_t* n_obs, double* batch, void* stream) {
  clear_error();
  if (R < 1 || K < 1 || K > 64) return fail(DSP_ERR_SHAPE, "need R >= 1 and 1 <= K <= 64 (R=%d K=%d)", R, K);
  if (n_bins < 1 || n_bins > kMaxBins) return fail(DSP_ERR_SHAPE, "n_bins must be in [1, 64] (got %d)", n_bins);
  if (ld_conf < K) return fail(DSP_ERR_SHAPE, "conf stride too small");
  if (!conf || !cu_seqlens || !decided || !ece || !n_obs || !batch)
    return fail(DSP_ERR_NULL, "required pointer is NULL");
  CalArgs a{conf, ld_conf, cu_seqlens, decided, R, K, n_bins, ece, n_obs, batch};
  launch(DSP_K_CALIBRATION, calibration_kernel, dim3(1), dim3(kCalThreads), 0, (hipStream_t)stream, a);
  return hip_check(hipGetLastError(), "calibration launch");
}
