// Confidence scheduler and ragged pack for gfx950.
//
// Scheduler (DSpark study notes, sections 5.1-5.2; SGLang article, "SPS cost
// table"): block survival S_{i,k} = prod_{j<=k} c_{i,j}; all candidates are
// ranked by S descending and taken greedily while expected throughput
// E / cost(N) strictly rises (non-anticipating early stop), or the smallest N
// maximising it (argmax mode). One workgroup of 1024 threads holds every
// candidate in LDS:
//   - survival in fp64 (one thread per request, left to right), quantised to
//     a 2^-Q grid and packed into a unique 64-bit key
//     ((2^41-1-Sq) << 23 | i << 7 | k-1) so ascending key order is
//     (S desc, i asc, k asc) and any correct sort gives the same order;
//   - bitonic sort (registers / wave shuffles / LDS by stride); exact uint64
//     prefix sums of Sq;
//   - the throughput test per candidate as two separate fp64 products
//     (E_j * c[j-1] > E_{j-1} * c[j]) and a block minimum for the first failure;
//   - window of request i = how many of its keys precede the first rejected key
//     (prefix closure makes this the count of taken candidates).
//
// Pack (SGLang article, "Ragged verify"): exclusive scan of n_i + 1, then each
// request writes its anchor and first n_i drafts front to back.
#include <math.h>

#include "dsp_internal.h"

namespace dsp {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kMaxCand = 8192;
constexpr uint64_t kInvMax = (1ull << 41) - 1;

__device__ __forceinline__ uint64_t sched_key(uint64_t sq, int i, int k0) {
  return ((kInvMax - sq) << 23) | ((uint64_t)i << 7) | (uint64_t)k0;
}
__device__ __forceinline__ uint64_t key_sq(uint64_t key) { return kInvMax - (key >> 23); }

__device__ __forceinline__ uint64_t quantise(double s, double scale) {
  return (uint64_t)floor(s * scale);
}

// Exclusive scan of one uint64 per thread over a 1024-thread block.
__device__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t run = 0;
    for (int j = 0; j < kSchedThreads / 64; ++j) {
      const uint64_t t = wsum[j];
      wsum[j] = run;
      run += t;
    }
  }
  __syncthreads();
  return wsum[w] + inc - v;
}

// Lane exchange at xor distance TS (1..32) inside a wavefront, with fixed patterns:
// DPP quad permutes for 1 and 2, ds_swizzle xor masks for 4, 8 and 16 (no LDS memory
// access), ds_bpermute only for 32.
template <int TS>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if (TS == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  if (TS == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  if (TS == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x101F);  // and 31, xor 4
  if (TS == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x201F);
  if (TS == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ 32) << 2), (int)x);
}
template <int TS, int E>
__device__ __forceinline__ void xor_lanes(const uint64_t* v, uint64_t* o) {
  uint32_t lo[E], hi[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    lo[e] = xor_lane<TS>((uint32_t)v[e]);
    hi[e] = xor_lane<TS>((uint32_t)(v[e] >> 32));
  }
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = ((uint64_t)hi[e] << 32) | lo[e];
}

// Ascending bitonic sort of keys[0..P) (P a power of two, 64 * E <= P <= 1024 * E) by
// the first P / E threads of a 1024-thread block, E consecutive keys per thread:
// strides below E are compare-exchanges in registers, strides below 64*E go through
// lane exchanges inside a wavefront (fixed patterns when E > 1), and only wider
// strides through LDS, so
// most of the log2(P)(log2(P)+1)/2 stages need neither memory nor a barrier.
template <int E>
__device__ void bitonic_keys(uint64_t* keys, int P) {
  const int tid = threadIdx.x;
  const bool act = tid * E < P;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = act ? keys[tid * E + e] : ~0ull;
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < E) {
        // partner in the same thread: element e ^ stride (stride in {1, 2, 4})
#pragma unroll
        for (int sb = 1; sb < E; sb <<= 1) {
          if (sb != stride) continue;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if (e & sb) continue;
            const bool up = ((tid * E + e) & size) == 0;
            const uint64_t a = v[e], b = v[e | sb];
            const bool sw = (a > b) == up;
            v[e] = sw ? b : a;
            v[e | sb] = sw ? a : b;
          }
        }
        continue;
      }
      const int ts = stride / E;  // distance in threads
      uint64_t o[E];
      if (ts < 64 && E == 1) {
        // one key per thread: a single lane permute costs less than a branch per stage
        o[0] = __shfl_xor(v[0], ts, 64);
      } else if (ts < 64) {
        // one uniform branch per stage, then straight-line fixed-pattern exchanges
        switch (ts) {
          case 1: xor_lanes<1, E>(v, o); break;
          case 2: xor_lanes<2, E>(v, o); break;
          case 4: xor_lanes<4, E>(v, o); break;
          case 8: xor_lanes<8, E>(v, o); break;
          case 16: xor_lanes<16, E>(v, o); break;
          default: xor_lanes<32, E>(v, o); break;
        }
      } else {
        __syncthreads();
        if (act)
#pragma unroll
          for (int e = 0; e < E; ++e) keys[tid * E + e] = v[e];
        __syncthreads();
        if (act)
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = keys[(tid ^ ts) * E + e];
      }
      const bool up = ((tid * E) & size) == 0;     // size > stride >= E: same for all e
      const bool low = ((tid * E) & stride) == 0;  // likewise
      const bool keep_min = low == up;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool lt = o[e] < v[e];
        v[e] = lt == keep_min ? o[e] : v[e];
      }
    }
  }
  __syncthreads();
  if (act)
#pragma unroll
    for (int e = 0; e < E; ++e) keys[tid * E + e] = v[e];
  __syncthreads();
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const float* __restrict__ conf, int R, int K, const double* __restrict__ cost, int mode, int M,
    double threshold, int Q, int32_t* __restrict__ windows, double* __restrict__ survival,
    double* __restrict__ stats) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ float s_conf[kMaxCand];
  __shared__ uint64_t wsum[kSchedThreads / 64];
  __shared__ double smd[kSchedThreads / 64];
  __shared__ int smi[kSchedThreads / 64];
  __shared__ uint64_t e_at_n;
  const int tid = threadIdx.x;
  const int n = R * K;
  int P = 1;
  while (P < n) P <<= 1;
  const double scale = ldexp(1.0, Q);

  // confidences staged in LDS with coalesced loads, then survival products and keys
  for (int j = tid; j < n; j += kSchedThreads) s_conf[j] = conf[j];
  __syncthreads();
  for (int i = tid; i < R; i += kSchedThreads) {
    double s = 1.0;
    for (int k = 0; k < K; ++k) {
      s = __dmul_rn(s, (double)s_conf[i * K + k]);
      if (survival) survival[(size_t)i * K + k] = s;
      keys[i * K + k] = sched_key(quantise(s, scale), i, k);
    }
  }
  for (int j = n + tid; j < (P < 64 ? 64 : P); j += kSchedThreads) keys[j] = ~0ull;
  __syncthreads();

  if (mode == DSP_SCHED_THRESHOLD) {
    // n_i = #{k : S_{i,k} >= threshold} on the fp64 survival; no ranking needed
    uint64_t esum = 0;
    int cnt_all = 0;
    for (int i = tid; i < R; i += kSchedThreads) {
      double s = 1.0;
      int cnt = 0;
      for (int k = 0; k < K; ++k) {
        s = __dmul_rn(s, (double)s_conf[i * K + k]);
        if (s >= threshold) {
          ++cnt;
          esum += quantise(s, scale);
        }
      }
      windows[i] = cnt;
      cnt_all += cnt;
    }
    const int Nt = block_sum<kSchedThreads / 64>(cnt_all, smi);
    const uint64_t Et = block_exclusive_scan_u64(esum, wsum) + esum;  // inclusive; the last thread holds the total
    if (stats && tid == kSchedThreads - 1) {
      const double E = ldexp((double)Et, -Q);
      stats[0] = (double)Nt;
      stats[1] = E;
      stats[2] = cost[Nt] != 0.0 ? __ddiv_rn(E, cost[Nt]) : (E == 0.0 ? 0.0 : INFINITY);
      stats[3] = (double)Q;
    }
    return;
  }

  // bitonic sort, ascending, over at least one full wavefront of slots (padding keys
  // are ~0 and sort last), with as many threads as the size allows
  const int PS = P < 64 ? 64 : P;
  if (PS <= 1024) bitonic_keys<1>(keys, PS);
  else if (PS == 2048) bitonic_keys<2>(keys, PS);
  else if (PS == 4096) bitonic_keys<4>(keys, PS);
  else bitonic_keys<8>(keys, PS);

  // exact prefix sums over the first M sorted candidates; thread t owns [t*C, t*C + C)
  const int C = (M + kSchedThreads - 1) / kSchedThreads;
  const int p0 = min(M, tid * C), p1 = min(M, p0 + C);
  uint64_t local = 0;
  for (int p = p0; p < p1; ++p) local += key_sq(keys[p]);
  const uint64_t ex = block_exclusive_scan_u64(local, wsum);

  int N;
  if (mode == DSP_SCHED_TOP_M) {
    N = M;  // a capacity decided earlier: the first M candidates of the current order
  } else if (mode == DSP_SCHED_EARLY_STOP) {
    int first_fail = 0x7fffffff;
    uint64_t run = ex;
    for (int p = p0; p < p1; ++p) {
      const int j = p + 1;
      const uint64_t Ej = run + key_sq(keys[p]);
      const double lhs = __dmul_rn((double)Ej, cost[j - 1]);
      const double rhs = __dmul_rn((double)run, cost[j]);
      if (!(lhs > rhs)) {
        first_fail = j;
        break;
      }
      run = Ej;
    }
    const int ff = block_min<kSchedThreads / 64>(first_fail, smi);
    N = ff == 0x7fffffff ? M : ff - 1;
  } else {
    double best = -1.0;
    int bj = 0x7fffffff;
    if (tid == 0) {
      best = __ddiv_rn(0.0, cost[0]);
      bj = 0;
    }
    uint64_t run = ex;
    for (int p = p0; p < p1; ++p) {
      const int j = p + 1;
      run += key_sq(keys[p]);
      const double J = __ddiv_rn((double)run, cost[j]);
      if (J > best) {
        best = J;
        bj = j;
      }
    }
    const double Jm = block_max<kSchedThreads / 64>(best, smd);
    const int jm = block_min<kSchedThreads / 64>(best == Jm ? bj : 0x7fffffff, smi);
    N = jm;
  }

  // E at N (sum of the first N quantised survivals)
  if (tid == 0) e_at_n = 0;
  __syncthreads();
  if (N > 0 && N - 1 >= p0 && N - 1 < p1) {
    uint64_t run = ex;
    for (int p = p0; p < N; ++p) run += key_sq(keys[p]);
    e_at_n = run;
  }
  __syncthreads();
  const uint64_t thr = N < n ? keys[N] : ~0ull;

  // window of request i: its candidates ranked before the first untaken one
  for (int i = tid; i < R; i += kSchedThreads) {
    double s = 1.0;
    int cnt = 0;
    for (int k = 0; k < K; ++k) {
      s = __dmul_rn(s, (double)s_conf[i * K + k]);
      cnt += sched_key(quantise(s, scale), i, k) < thr ? 1 : 0;
    }
    windows[i] = cnt;
  }
  if (stats && tid == 0) {
    const double E = ldexp((double)e_at_n, -Q);
    stats[0] = (double)N;
    stats[1] = E;
    stats[2] = cost[N] != 0.0 ? __ddiv_rn(E, cost[N]) : (E == 0.0 ? 0.0 : INFINITY);
    stats[3] = (double)Q;
  }
}

struct Tiers {
  int32_t n;
  int32_t v[64];
};

__global__ __launch_bounds__(1024) void pack_kernel(const int32_t* __restrict__ windows,
                                                    const int32_t* __restrict__ anchors,
                                                    const int32_t* __restrict__ drafts, int64_t ld,
                                                    int R, int K, Tiers tiers, int32_t* __restrict__ cu,
                                                    int32_t* __restrict__ tokens,
                                                    int32_t* __restrict__ row_req,
                                                    int32_t* __restrict__ row_pos,
                                                    int32_t* __restrict__ total_and_tier,
                                                    int32_t* __restrict__ status) {
  __shared__ uint64_t wsum[16];
  const int tid = threadIdx.x;
  const int C = (R + 1023) / 1024;
  const int i0 = min(R, tid * C), i1 = min(R, i0 + C);
  uint64_t local = 0;
  bool bad = false;
  for (int i = i0; i < i1; ++i) {
    int w = windows[i];
    if (w < 0 || w > K) {
      bad = true;
      w = w < 0 ? 0 : K;
    }
    local += (uint64_t)(w + 1);
  }
  if (bad) atomicOr(status, DSP_STATUS_WINDOW_RANGE);
  const uint64_t ex = block_exclusive_scan_u64(local, wsum);
  // offsets first (each thread its own requests), then one flat copy over (request, position)
  int pos = (int)ex;
  if (tid == 0) cu[0] = 0;
  for (int i = i0; i < i1; ++i) {
    int w = windows[i];
    w = w < 0 ? 0 : (w > K ? K : w);
    pos += w + 1;
    cu[i + 1] = pos;
  }
  if (i1 == R && i0 < i1) {
    const int T = pos;
    int tier = T;
    if (tiers.n > 0) {
      tier = -1;
      for (int t = 0; t < tiers.n; ++t)
        if (tiers.v[t] >= T) {
          tier = tiers.v[t];
          break;
        }
    }
    total_and_tier[0] = T;
    total_and_tier[1] = tier;
  }
  __threadfence_block();
  __syncthreads();
  const int K1 = K + 1;
  for (long j = tid; j < (long)R * K1; j += 1024) {
    const int i = (int)(j / K1), k = (int)(j % K1);
    const int start = cu[i];
    if (start + k >= cu[i + 1]) continue;  // beyond this request's window
    tokens[start + k] = k == 0 ? anchors[i] : drafts[(size_t)i * ld + k - 1];
    row_req[start + k] = i;
    row_pos[start + k] = k;
  }
}

int quant_bits(int R, int K) {
  long n = (long)R * K;
  int c = 0;
  while ((1l << c) < n) ++c;  // ceil(log2 n)
  const int q = 53 - c;
  return q < 40 ? q : 40;
}

}  // namespace
}  // namespace dsp

using namespace dsp;

extern "C" size_t dsp_schedule_windows_workspace_size(int32_t R, int32_t K) {
  (void)R;
  (void)K;
  return 0;
}

extern "C" int32_t dsp_schedule_windows(const float* conf, int32_t R, int32_t K, const double* cost,
                                        int32_t n_cost, int32_t mode, int32_t max_tokens, double threshold,
                                        int32_t* windows, double* survival, double* stats, void* ws,
                                        size_t ws_bytes, void* stream) {
  clear_error();
  (void)ws;
  (void)ws_bytes;
  if (R < 1 || K < 1 || K > 128 || (long)R * K > kMaxCand)
    return fail(DSP_ERR_SHAPE, "need R >= 1, 1 <= K <= 128, R*K <= %d (R=%d K=%d)", kMaxCand, R, K);
  if (n_cost < R * K + 1) return fail(DSP_ERR_SHAPE, "cost table needs R*K+1 = %d entries", R * K + 1);
  if (mode != DSP_SCHED_EARLY_STOP && mode != DSP_SCHED_ARGMAX && mode != DSP_SCHED_TOP_M &&
      mode != DSP_SCHED_THRESHOLD)
    return fail(DSP_ERR_UNSUPPORTED, "unknown scheduler mode %d", mode);
  if (mode == DSP_SCHED_THRESHOLD && !(threshold == threshold))
    return fail(DSP_ERR_SHAPE, "threshold must not be NaN");
  if (!conf || !cost || !windows) return fail(DSP_ERR_NULL, "conf, cost and windows are required");
  const int M = max_tokens < 0 ? R * K : (max_tokens < R * K ? max_tokens : R * K);
  launch(DSP_K_SCHEDULE, schedule_kernel, dim3(1), dim3(kSchedThreads), 0, (hipStream_t)stream, conf, R, K,
         cost, mode, M, threshold, quant_bits(R, K), windows, survival, stats);
  return hip_check(hipGetLastError(), "schedule launch");
}

extern "C" int32_t dsp_pack_ragged(const int32_t* windows, const int32_t* anchors, const int32_t* drafts,
                                   int64_t ld_drafts, int32_t R, int32_t K, const int32_t* tiers_host,
                                   int32_t n_tiers, int32_t* cu_seqlens, int32_t* tokens,
                                   int32_t* row_req, int32_t* row_pos, int32_t* total_and_tier,
                                   int32_t* status, void* stream) {
  clear_error();
  if (R < 1 || R > 65536 || K < 1 || K > 4096) return fail(DSP_ERR_SHAPE, "need 1 <= R <= 65536, 1 <= K <= 4096");
  if (ld_drafts < K) return fail(DSP_ERR_SHAPE, "ld_drafts < K");
  if (n_tiers < 0 || n_tiers > 64 || (n_tiers > 0 && !tiers_host))
    return fail(DSP_ERR_SHAPE, "n_tiers must be in [0, 64] with a host tier array");
  if (!windows || !anchors || !drafts || !cu_seqlens || !tokens || !row_req || !row_pos ||
      !total_and_tier || !status)
    return fail(DSP_ERR_NULL, "required pointer is NULL");
  Tiers t;
  t.n = n_tiers;
  for (int j = 0; j < 64; ++j) t.v[j] = j < n_tiers ? tiers_host[j] : 0;
  for (int j = 1; j < n_tiers; ++j)
    if (t.v[j] < t.v[j - 1]) return fail(DSP_ERR_SHAPE, "tiers must be ascending");
  launch(DSP_K_PACK, pack_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, windows, anchors, drafts,
         ld_drafts, R, K, t, cu_seqlens, tokens, row_req, row_pos, total_and_tier, status);
  return hip_check(hipGetLastError(), "pack launch");
}
