// Confidence scheduler and ragged pack for gfx950.
//
// Scheduler (DSpark study notes, sections 5.1-5.2; SGLang article, "SPS cost
// table"): block survival S_{i,k} = prod_{j<=k} c_{i,j}; all candidates are
// ranked by S descending and taken greedily while expected throughput
// E / cost(N) strictly rises (non-anticipating early stop), or the smallest N
// maximising it (argmax mode). Two launches:
//   - ranking, over many workgroups: each builds every candidate key in LDS --
//     survival in fp64 (one thread per request, left to right), quantised to a
//     2^-Q grid and packed into a unique 64-bit key ((2^41-1-Sq) << 23 | i << 7
//     | k-1), so ascending key order is (S desc, i asc, k asc) -- and places a
//     few of them at their rank (the number of smaller keys, counted by brute
//     force: n^2 compares spread over the chip cost less than any sort in one
//     workgroup);
//   - selection, one workgroup of 1024 threads: exact uint64 prefix sums of Sq,
//     the throughput test per candidate as two separate fp64 products
//     (E_j * c[j-1] > E_{j-1} * c[j]) with a block minimum for the first
//     failure, and window of request i = how many of its candidates are taken.
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
  // every thread adds up the waves before its own (16 independent LDS reads, no serial
  // pass by one thread)
  uint64_t pre = 0;
#pragma unroll
  for (int j = 0; j < kSchedThreads / 64; ++j) pre += j < w ? wsum[j] : 0ull;
  __syncthreads();  // wsum may be reused by the next scan
  return pre + inc - v;
}

// conf [n] into LDS: 32 loads per thread in flight per round (clamped, stored only in
// range), so a whole table of up to 32 x blockDim entries takes one round trip.
__device__ __forceinline__ void stage_conf(const float* __restrict__ conf, int n, float* s_conf) {
  for (int j0 = threadIdx.x; j0 < n; j0 += 32 * blockDim.x) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) v[q] = conf[min(j0 + q * (int)blockDim.x, n - 1)];
#pragma unroll
    for (int q = 0; q < 32; ++q)
      if (j0 + q * (int)blockDim.x < n) s_conf[j0 + q * blockDim.x] = v[q];
  }
}

// The ranking reads the keys kKeyBlock at a time; kMaxCand is a multiple of it.
constexpr int kKeyBlock = 512;
static_assert(kMaxCand % kKeyBlock == 0, "padded keys must fit the key table");

// Candidate keys of every (request, position): survival in fp64, one thread per
// request multiplying left to right, quantised and packed (optionally also written
// out as the survival table). Each thread reads its own request's confidences straight
// from global memory, sixteen in flight per round (as four 16-byte loads when the rows
// are 16-byte aligned), and the keys are stored position-major, keys[k * R + i], so the
// lanes of a wave write consecutive words; the ranking counts over all keys, so their
// order in LDS does not matter.
__device__ void candidate_keys(const float* __restrict__ conf, int R, int K, double scale, uint64_t* keys,
                               double* survival) {
  const int n = R * K;
  const bool v4 = (K & 3) == 0 && ((uintptr_t)conf & 15) == 0;
  for (int i = threadIdx.x; i < R; i += blockDim.x) {
    const float* row = conf + (size_t)i * K;
    double s = 1.0;
    for (int k0 = 0; k0 < K; k0 += 16) {
      float cf[16];
      if (v4 && k0 + 16 <= K) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = *(const float4*)(row + k0 + 4 * q);
          cf[4 * q] = t.x, cf[4 * q + 1] = t.y, cf[4 * q + 2] = t.z, cf[4 * q + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) cf[q] = k0 + q < K ? row[k0 + q] : 1.0f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int k = k0 + q;
        if (k < K) {
          s = __dmul_rn(s, (double)cf[q]);
          if (survival) survival[(size_t)i * K + k] = s;
          keys[k * R + i] = sched_key(quantise(s, scale), i, k);
        }
      }
    }
  }
  // padding keys (never below a real key) up to a whole number of kKeyBlock-key blocks
  for (int j = n + threadIdx.x; j < ((n + kKeyBlock - 1) & ~(kKeyBlock - 1)); j += blockDim.x) keys[j] = ~0ull;
  __syncthreads();
}

// Ranking, spread over many workgroups: each workgroup builds every key in LDS and
// ranks kRankCand of them by counting the keys below each (keys are unique, so the
// counts are a permutation of 0..n-1), kRankSlices lanes per candidate over
// interleaved slices of the keys: slice s reads key pairs (2s, 2s+1) of every strip of
// 2*kRankSlices keys (lanes of one slice read the same LDS words: a broadcast), the
// kRankReads strips of a kKeyBlock-key block per step. 1024 threads give every SIMD
// four waves, so one wave's compares run while another waits on its LDS reads. The
// sorted keys go to sorted[rank].
constexpr int kRankThreads = 1024;
constexpr int kSelPer = kMaxCand / kSchedThreads;  // ranks per thread in the selection
constexpr int kRankCand = 16;
constexpr int kRankSlices = kRankThreads / kRankCand;
constexpr int kRankReads = kKeyBlock / (2 * kRankSlices);
static_assert(kRankReads * 2 * kRankSlices == kKeyBlock, "slices must tile a key block");

__global__ __launch_bounds__(kRankThreads) void schedule_rank_kernel(const float* __restrict__ conf, int R,
                                                                     int K, int Q, double* __restrict__ survival,
                                                                     uint64_t* __restrict__ sorted) {
  __shared__ __align__(16) uint64_t keys[kMaxCand];
  __shared__ __align__(16) int part[kRankThreads];
  const int tid = threadIdx.x;
  const int n = R * K;
  candidate_keys(conf, R, K, ldexp(1.0, Q), keys, blockIdx.x == 0 ? survival : nullptr);
  const int cl = tid % kRankCand, sl = tid / kRankCand;
  const int c = blockIdx.x * kRankCand + cl;
  const uint64_t x = c < n ? keys[c] : 0ull;
  int cnt = 0;
  const int np = (n + kKeyBlock - 1) & ~(kKeyBlock - 1);  // padded with keys above every real one
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  for (int j = 2 * sl; j < np; j += kKeyBlock) {  // kRankReads reads in flight per round
    u64x2 v[kRankReads];
#pragma unroll
    for (int q = 0; q < kRankReads; ++q) v[q] = *(const u64x2*)&keys[j + 2 * kRankSlices * q];
#pragma unroll
    for (int q = 0; q < kRankReads; ++q) cnt += (v[q].x < x ? 1 : 0) + (v[q].y < x ? 1 : 0);
  }
  part[cl * kRankSlices + sl] = cnt;  // a candidate's partial counts side by side
  __syncthreads();
  if (sl == 0 && c < n) {
    int r = 0;
#pragma unroll
    for (int q = 0; q < kRankSlices; ++q) r += part[cl * kRankSlices + q];
    sorted[r] = x;
  }
}

struct Tiers {
  int32_t n;
  int32_t v[64];
};

// The pack outputs (and its inputs besides the windows).
struct PackArgs {
  const int32_t* anchors;
  const int32_t* drafts;
  int64_t ld;
  Tiers tiers;
  int32_t* cu;
  int32_t* tokens;
  int32_t* row_req;
  int32_t* row_pos;
  int32_t* total_and_tier;
  int32_t* status;
};

// The pack, run by one workgroup of 1024 threads over windows already in memory (wsum:
// 16 LDS words for the scan).
__device__ void pack_body(const int32_t* __restrict__ windows, int R, int K, const PackArgs& pa, uint64_t* wsum) {
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
  if (bad) atomicOr(pa.status, DSP_STATUS_WINDOW_RANGE);
  const uint64_t ex = block_exclusive_scan_u64(local, wsum);
  // offsets first (each thread its own requests), then one flat copy over (request, position)
  int pos = (int)ex;
  if (tid == 0) pa.cu[0] = 0;
  for (int i = i0; i < i1; ++i) {
    int w = windows[i];
    w = w < 0 ? 0 : (w > K ? K : w);
    pos += w + 1;
    pa.cu[i + 1] = pos;
  }
  if (i1 == R && i0 < i1) {
    const int T = pos;
    int tier = T;
    if (pa.tiers.n > 0) {
      tier = -1;
      for (int t = 0; t < pa.tiers.n; ++t)
        if (pa.tiers.v[t] >= T) {
          tier = pa.tiers.v[t];
          break;
        }
    }
    pa.total_and_tier[0] = T;
    pa.total_and_tier[1] = tier;
  }
  __threadfence_block();
  __syncthreads();
  const int K1 = K + 1;
  for (long j = tid; j < (long)R * K1; j += 1024) {
    const int i = (int)(j / K1), k = (int)(j % K1);
    const int start = pa.cu[i];
    if (start + k >= pa.cu[i + 1]) continue;  // beyond this request's window
    pa.tokens[start + k] = k == 0 ? pa.anchors[i] : pa.drafts[(size_t)i * pa.ld + k - 1];
    pa.row_req[start + k] = i;
    pa.row_pos[start + k] = k;
  }
}

// The pack inside the selection workgroup (R*K <= kMaxCand): every token it may copy is
// loaded up front (pack_prefetch, issued at the start of the selection so the loads
// overlap it), the windows come from LDS and the offsets stay in LDS, so the copy needs
// no further round trip to memory. Thread t holds items t, t + 1024, ... of the
// (request, position) grid R x (K+1), position 0 being the anchor.
constexpr int kPackPre = 2 * kMaxCand / kSchedThreads;  // R*(K+1) <= 2*R*K
// (request, position) of item j of the R x (K+1) grid without an integer division:
// (j + 1/2) / (K+1) is at least 1/(2(K+1)) >= 1/258 away from an integer, and the float
// quotient of j < 2^15 errs by less than 2^-8, so truncation gives the exact quotient.
__device__ __forceinline__ void pack_item(int j, int K1, float inv_k1, int& i, int& k) {
  i = (int)(((float)j + 0.5f) * inv_k1);
  k = j - i * K1;
}
__device__ void pack_prefetch(int R, int K, const PackArgs& pa, int32_t (&tok)[kPackPre]) {
  const int K1 = K + 1, n = R * K1, tid = threadIdx.x;
  const float inv_k1 = 1.0f / (float)K1;
  const int rounds = (n + kSchedThreads - 1) / kSchedThreads;  // the same in every thread
#pragma unroll
  for (int q = 0; q < kPackPre; ++q) {  // clamped items (masked at use): all loads in flight at once
    if (q < rounds) {
      const int j = min(tid + q * kSchedThreads, n - 1);
      int i, k;
      pack_item(j, K1, inv_k1, i, k);
      // the source picked by address, so every item costs one load and no branch
      const int32_t* src = k == 0 ? pa.anchors + i : pa.drafts + ((size_t)i * pa.ld + (k > 0 ? k - 1 : 0));
      tok[q] = *src;
    }
  }
}
__device__ void pack_body_lds(const int* s_win, int R, int K, const PackArgs& pa, uint64_t* wsum, int* s_cu,
                              const int32_t (&tok)[kPackPre]) {
  const int tid = threadIdx.x;
  const int C = (R + kSchedThreads - 1) / kSchedThreads;
  const int i0 = min(R, tid * C), i1 = min(R, i0 + C);
  uint64_t local = 0;
  bool bad = false;
  for (int i = i0; i < i1; ++i) {
    int w = s_win[i];
    if (w < 0 || w > K) {
      bad = true;
      w = w < 0 ? 0 : K;
    }
    local += (uint64_t)(w + 1);
  }
  if (bad) atomicOr(pa.status, DSP_STATUS_WINDOW_RANGE);
  const uint64_t ex = block_exclusive_scan_u64(local, wsum);
  int pos = (int)ex;
  if (tid == 0) {
    pa.cu[0] = 0;
    s_cu[0] = 0;
  }
  for (int i = i0; i < i1; ++i) {
    int w = s_win[i];
    w = w < 0 ? 0 : (w > K ? K : w);
    pos += w + 1;
    pa.cu[i + 1] = pos;
    s_cu[i + 1] = pos;
  }
  if (i1 == R && i0 < i1) {
    const int T = pos;
    int tier = T;
    if (pa.tiers.n > 0) {
      tier = -1;
      for (int t = 0; t < pa.tiers.n; ++t)
        if (pa.tiers.v[t] >= T) {
          tier = pa.tiers.v[t];
          break;
        }
    }
    pa.total_and_tier[0] = T;
    pa.total_and_tier[1] = tier;
  }
  __syncthreads();
  const int K1 = K + 1, n = R * K1;
  const float inv_k1 = 1.0f / (float)K1;
#pragma unroll
  for (int q = 0; q < kPackPre; ++q) {
    const int j = tid + q * kSchedThreads;
    if (j >= n) break;
    int i, k;
    pack_item(j, K1, inv_k1, i, k);
    const int start = s_cu[i];
    if (start + k >= s_cu[i + 1]) continue;  // beyond this request's window
    pa.tokens[start + k] = tok[q];
    pa.row_req[start + k] = i;
    pa.row_pos[start + k] = k;
  }
}

__global__ __launch_bounds__(1024) void pack_kernel(const int32_t* __restrict__ windows, int R, int K,
                                                    PackArgs pa) {
  __shared__ uint64_t wsum[16];
  pack_body(windows, R, K, pa, wsum);
}

// Selection over the ranked keys (one workgroup): exact prefix sums of Sq, the
// throughput test, E at N, and the windows; or the fixed-threshold rule straight
// from the survivals (then no ranking is needed and sorted is unused).
__global__ __launch_bounds__(kSchedThreads) void schedule_select_kernel(
    const float* __restrict__ conf, int R, int K, const double* __restrict__ cost, int mode, int M,
    double threshold, int Q, const uint64_t* __restrict__ sorted, int32_t* __restrict__ windows,
    double* __restrict__ survival, double* __restrict__ stats, PackArgs pa) {
  __shared__ float s_conf[kMaxCand + 1];  // threshold mode; then the pack's R + 1 offsets
  __shared__ int cnt[kMaxCand];
  __shared__ uint64_t wsum[kSchedThreads / 64];
  __shared__ double smd[kSchedThreads / 64];
  __shared__ int smi[kSchedThreads / 64];
  __shared__ uint64_t e_at_n;
  const int tid = threadIdx.x;
  const int n = R * K;
  const double scale = ldexp(1.0, Q);
  int32_t tok[kPackPre];
  if (pa.cu) pack_prefetch(R, K, pa, tok);  // in flight during the selection
  int* s_cu = (int*)s_conf;                  // the pack's offsets (s_conf is free by then)

  if (mode == DSP_SCHED_THRESHOLD) {
    // n_i = #{k : S_{i,k} >= threshold} on the fp64 survival; no ranking needed
    stage_conf(conf, n, s_conf);
    __syncthreads();
    uint64_t esum = 0;
    int cnt_all = 0;
    for (int i = tid; i < R; i += kSchedThreads) {
      double s = 1.0;
      int c = 0;
      for (int k = 0; k < K; ++k) {
        s = __dmul_rn(s, (double)s_conf[i * K + k]);
        if (survival) survival[(size_t)i * K + k] = s;
        if (s >= threshold) {
          ++c;
          esum += quantise(s, scale);
        }
      }
      windows[i] = c;
      cnt[i] = c;
      cnt_all += c;
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
    if (pa.cu) {  // the pack of these windows, in this workgroup
      __syncthreads();
      pack_body_lds(cnt, R, K, pa, wsum, s_cu, tok);
    }
    return;
  }

  // thread t owns ranks [t*C, t*C + C) of the first M (C <= kSelPer): its keys and the
  // cost entries it needs are loaded straight into registers, all in one round trip.
  // The trip count C is the same in every thread and the indices are clamped, so no
  // load sits under a per-lane branch; entries past p1 are masked at every use.
  const int C = (M + kSchedThreads - 1) / kSchedThreads;
  const int p0 = min(M, tid * C), p1 = min(M, p0 + C);
  uint64_t kq[kSelPer];
  double cq[kSelPer + 1];
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) kq[q] = q < C ? sorted[min(p0 + q, M - 1)] : 0ull;
#pragma unroll
  for (int q = 0; q <= kSelPer; ++q) cq[q] = q <= C ? cost[min(p0 + q, M)] : 0.0;
  for (int i = tid; i < R; i += kSchedThreads) cnt[i] = 0;

  // exact prefix sums of the quantised survivals in rank order
  uint64_t local = 0;
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) local += p0 + q < p1 ? key_sq(kq[q]) : 0ull;
  const uint64_t ex = block_exclusive_scan_u64(local, wsum);

  int N;
  if (mode == DSP_SCHED_TOP_M) {
    N = M;  // a capacity decided earlier: the first M candidates of the current order
  } else if (mode == DSP_SCHED_EARLY_STOP) {
    int first_fail = 0x7fffffff;
    uint64_t run = ex;
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) {
      if (p0 + q < p1 && first_fail == 0x7fffffff) {
        const int j = p0 + q + 1;
        const uint64_t Ej = run + key_sq(kq[q]);
        const double lhs = __dmul_rn((double)Ej, cq[q]);       // E_j * c[j-1]
        const double rhs = __dmul_rn((double)run, cq[q + 1]);  // E_{j-1} * c[j]
        if (!(lhs > rhs)) first_fail = j;
        run = Ej;
      }
    }
    const int ff = block_min<kSchedThreads / 64>(first_fail, smi);
    N = ff == 0x7fffffff ? M : ff - 1;
  } else {
    double best = -1.0;
    int bj = 0x7fffffff;
    if (tid == 0) {
      best = __ddiv_rn(0.0, cq[0]);
      bj = 0;
    }
    // the C quotients first (independent, so their division sequences overlap), then
    // the comparisons in rank order over the valid ones
    uint64_t run = ex;
    double Jq[kSelPer];
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) {
      if (q < C) {
        run += key_sq(kq[q]);
        Jq[q] = __ddiv_rn((double)run, cq[q + 1]);
      }
    }
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) {
      if (q < C && p0 + q < p1 && Jq[q] > best) {
        best = Jq[q];
        bj = p0 + q + 1;
      }
    }
    const double Jm = block_max<kSchedThreads / 64>(best, smd);
    const int jm = block_min<kSchedThreads / 64>(best == Jm ? bj : 0x7fffffff, smi);
    N = jm;
  }

  // E at N (sum of the first N quantised survivals), and the window of request i: how
  // many of its candidates are among the first N (its taken candidates are its leading
  // positions whenever the survival does not grow along k)
  if (N > 0 && N - 1 >= p0 && N - 1 < p1) {
    uint64_t run = ex;
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) run += p0 + q < N ? key_sq(kq[q]) : 0ull;  // N <= p1 here
    e_at_n = run;
  }
  if (N == 0 && tid == 0) e_at_n = 0;
#pragma unroll
  for (int q = 0; q < kSelPer; ++q)
    if (p0 + q < p1 && p0 + q < N) atomicAdd(&cnt[(int)((kq[q] >> 7) & 0xFFFFu)], 1);
  __syncthreads();
  for (int i = tid; i < R; i += kSchedThreads) windows[i] = cnt[i];
  if (stats && tid == 0) {
    const double E = ldexp((double)e_at_n, -Q);
    stats[0] = (double)N;
    stats[1] = E;
    stats[2] = cost[N] != 0.0 ? __ddiv_rn(E, cost[N]) : (E == 0.0 ? 0.0 : INFINITY);
    stats[3] = (double)Q;
  }
  if (pa.cu) {  // the pack of these windows, in this workgroup (windows from LDS)
    __syncthreads();
    pack_body_lds(cnt, R, K, pa, wsum, s_cu, tok);
  }
}

// Validates the pack's arguments (windows apart) and fills pa; 0 or an error code.
int32_t pack_args(const int32_t* anchors, const int32_t* drafts, int64_t ld_drafts, int32_t R, int32_t K,
                  const int32_t* tiers_host, int32_t n_tiers, int32_t* cu_seqlens, int32_t* tokens,
                  int32_t* row_req, int32_t* row_pos, int32_t* total_and_tier, int32_t* status, PackArgs* pa) {
  if (R < 1 || R > 65536 || K < 1 || K > 4096) return fail(DSP_ERR_SHAPE, "need 1 <= R <= 65536, 1 <= K <= 4096");
  if (ld_drafts < K) return fail(DSP_ERR_SHAPE, "ld_drafts < K");
  if (n_tiers < 0 || n_tiers > 64 || (n_tiers > 0 && !tiers_host))
    return fail(DSP_ERR_SHAPE, "n_tiers must be in [0, 64] with a host tier array");
  if (!anchors || !drafts || !cu_seqlens || !tokens || !row_req || !row_pos || !total_and_tier || !status)
    return fail(DSP_ERR_NULL, "required pointer is NULL");
  pa->anchors = anchors;
  pa->drafts = drafts;
  pa->ld = ld_drafts;
  pa->tiers.n = n_tiers;
  for (int j = 0; j < 64; ++j) pa->tiers.v[j] = j < n_tiers ? tiers_host[j] : 0;
  for (int j = 1; j < n_tiers; ++j)
    if (pa->tiers.v[j] < pa->tiers.v[j - 1]) return fail(DSP_ERR_SHAPE, "tiers must be ascending");
  pa->cu = cu_seqlens;
  pa->tokens = tokens;
  pa->row_req = row_req;
  pa->row_pos = row_pos;
  pa->total_and_tier = total_and_tier;
  pa->status = status;
  return DSP_OK;
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
  if (R < 1 || K < 1) return 0;
  return ((size_t)R * K * sizeof(uint64_t) + 255) & ~(size_t)255;  // the ranked keys
}

namespace dsp {
namespace {
// Validates the scheduler's arguments; 0 or an error code.
int32_t schedule_check(const float* conf, int32_t R, int32_t K, const double* cost, int32_t n_cost, int32_t mode,
                       double threshold, int32_t* windows, void* ws, size_t ws_bytes) {
  if (R < 1 || K < 1 || K > 128 || (long)R * K > kMaxCand)
    return fail(DSP_ERR_SHAPE, "need R >= 1, 1 <= K <= 128, R*K <= %d (R=%d K=%d)", kMaxCand, R, K);
  if (n_cost < R * K + 1) return fail(DSP_ERR_SHAPE, "cost table needs R*K+1 = %d entries", R * K + 1);
  if (mode != DSP_SCHED_EARLY_STOP && mode != DSP_SCHED_ARGMAX && mode != DSP_SCHED_TOP_M &&
      mode != DSP_SCHED_THRESHOLD)
    return fail(DSP_ERR_UNSUPPORTED, "unknown scheduler mode %d", mode);
  if (mode == DSP_SCHED_THRESHOLD && !(threshold == threshold))
    return fail(DSP_ERR_SHAPE, "threshold must not be NaN");
  if (!conf || !cost || !windows) return fail(DSP_ERR_NULL, "conf, cost and windows are required");
  if (!ws || ws_bytes < dsp_schedule_windows_workspace_size(R, K))
    return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", dsp_schedule_windows_workspace_size(R, K));
  return DSP_OK;
}

// The scheduler's launches; with pa.cu set, the selection workgroup also packs.
int32_t schedule_launch(const float* conf, int32_t R, int32_t K, const double* cost, int32_t mode,
                        int32_t max_tokens, double threshold, int32_t* windows, double* survival, double* stats,
                        void* ws, const PackArgs& pa, hipStream_t s) {
  const int M = max_tokens < 0 ? R * K : (max_tokens < R * K ? max_tokens : R * K);
  const int Q = quant_bits(R, K);
  uint64_t* sorted = (uint64_t*)ws;
  if (mode != DSP_SCHED_THRESHOLD) {
    const int g = (R * K + kRankCand - 1) / kRankCand;
    launch(DSP_K_SCHEDULE_RANK, schedule_rank_kernel, dim3(g), dim3(kRankThreads), 0, s, conf, R, K, Q, survival,
           sorted);
  }
  launch(DSP_K_SCHEDULE, schedule_select_kernel, dim3(1), dim3(kSchedThreads), 0, s, conf, R, K, cost, mode, M,
         threshold, Q, (const uint64_t*)sorted, windows, survival, stats, pa);
  return hip_check(hipGetLastError(), "schedule launch");
}
}  // namespace
}  // namespace dsp

extern "C" int32_t dsp_schedule_windows(const float* conf, int32_t R, int32_t K, const double* cost,
                                        int32_t n_cost, int32_t mode, int32_t max_tokens, double threshold,
                                        int32_t* windows, double* survival, double* stats, void* ws,
                                        size_t ws_bytes, void* stream) {
  clear_error();
  const int32_t rc = schedule_check(conf, R, K, cost, n_cost, mode, threshold, windows, ws, ws_bytes);
  if (rc) return rc;
  PackArgs none{};
  return schedule_launch(conf, R, K, cost, mode, max_tokens, threshold, windows, survival, stats, ws, none,
                         (hipStream_t)stream);
}

extern "C" int32_t dsp_schedule_pack(const float* conf, int32_t R, int32_t K, const double* cost, int32_t n_cost,
                                     int32_t mode, int32_t max_tokens, double threshold, int32_t* windows,
                                     double* survival, double* stats, const int32_t* anchors,
                                     const int32_t* drafts, int64_t ld_drafts, const int32_t* tiers_host,
                                     int32_t n_tiers, int32_t* cu_seqlens, int32_t* tokens, int32_t* row_req,
                                     int32_t* row_pos, int32_t* total_and_tier, int32_t* status, void* ws,
                                     size_t ws_bytes, void* stream) {
  clear_error();
  int32_t rc = schedule_check(conf, R, K, cost, n_cost, mode, threshold, windows, ws, ws_bytes);
  if (rc) return rc;
  PackArgs pa{};
  rc = pack_args(anchors, drafts, ld_drafts, R, K, tiers_host, n_tiers, cu_seqlens, tokens, row_req, row_pos,
                 total_and_tier, status, &pa);
  if (rc) return rc;
  return schedule_launch(conf, R, K, cost, mode, max_tokens, threshold, windows, survival, stats, ws, pa,
                         (hipStream_t)stream);
}

extern "C" int32_t dsp_pack_ragged(const int32_t* windows, const int32_t* anchors, const int32_t* drafts,
                                   int64_t ld_drafts, int32_t R, int32_t K, const int32_t* tiers_host,
                                   int32_t n_tiers, int32_t* cu_seqlens, int32_t* tokens,
                                   int32_t* row_req, int32_t* row_pos, int32_t* total_and_tier,
                                   int32_t* status, void* stream) {
  clear_error();
  if (!windows) return fail(DSP_ERR_NULL, "required pointer is NULL");
  PackArgs pa{};
  const int32_t rc = pack_args(anchors, drafts, ld_drafts, R, K, tiers_host, n_tiers, cu_seqlens, tokens, row_req,
                               row_pos, total_and_tier, status, &pa);
  if (rc) return rc;
  launch(DSP_K_PACK, pack_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, windows, R, K, pa);
  return hip_check(hipGetLastError(), "pack launch");
}
