// Batched ragged verify for gfx950.
//
// Operation (DSpark study notes, section 1 and Figure 1; SGLang article,
// "three verify modes" and "Ragged verify"; PCTree article for the greedy tree
// walk): per request, accept draft k with probability min(1, p_k(x_k)/q_k(x_k))
// left to right, stop at the first rejection and draw the corrected token from
// norm(max(0, p_k - q_k)), or draw the bonus token from p_{n+1} when the whole
// window is accepted. T = 0 is greedy matching; a parent array selects the
// greedy walk of a draft tree.
//
// Sampled path (T > 0), four launches on the caller's stream:
//   1. stats -- one streaming pass over every packed target row and every
//      windowed draft row. A workgroup owns a (row, chunk) item: up to 2048
//      16-byte loads in flight, the chunk maximum, then the sum of
//      exp2(x*c - ref) with ref = max*c (c = log2(e)/T): fp32 per element, fp64
//      across vectors. Items past the device-side packed total exit at once, so
//      ragged totals known only on the device need no host synchronisation.
//   2. decide -- one wavefront per request (lane k-1 = position k): merges the
//      chunk statistics into log-sum-exp (fp64), forms ratio = exp2(lp2 - lq2)
//      in fp64 with the Philox uniforms, finds the first rejection by ballot,
//      writes the accepted tokens and leaves a job (row, both log-sum-exps,
//      uniform) for the correction draw.
//   3. residual -- per (request, chunk): the fp64 mass of max(0, p - q) (or of
//      p for a bonus draw) over the chunk.
//   4. sample -- one workgroup per request: picks the chunk that holds
//      u' * total, rescans it with contiguous per-thread ranges and an fp64
//      exclusive scan, and writes the smallest token whose running sum exceeds
//      the target (the last positive entry if rounding leaves none).
// When the requests alone fill the chip (R >= 3/4 of the CUs), launches 2-4 are one
// launch instead: a 1024-thread workgroup per request decides with its first
// wavefront, streams the job's row(s) once into per-chunk masses in LDS and draws
// (one CU per request is then no loss, and no hand-off between launches is needed).
// No workgroup waits on another inside a kernel: on this chip the L2 is per
// XCD, and publishing data between workgroups would need an L2 write-back per
// hand-off, so every dependency is a kernel boundary instead.
//
// Greedy and tree paths: an arg-max streaming pass (lowest index on ties),
// then one wavefront per request for matching or the tree walk.
#include <math.h>

#include <mutex>

#include "dsp_internal.h"

namespace dsp {
namespace {

constexpr int kThreads = 256;
constexpr int kVpt = 8;                      // 16-byte vectors per thread per chunk (4 and 12-16 measured slower)
constexpr int kChunkVecs = kThreads * kVpt;  // vectors per chunk (2048 = 32 KiB of bf16)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct StatSlot {
  float ref;      // chunk max times c (fp32), or -inf for an empty chunk
  uint32_t flag;  // 1: chunk max not finite
  double sum;     // sum over the chunk of exp2(x*c - ref)
};
static_assert(sizeof(StatSlot) == 16, "slot size");

enum : int32_t { JOB_NONE = 0, JOB_RESID = 1, JOB_BONUS = 2 };

struct Job {
  int32_t mode;
  int32_t kstop;     // 1-based position whose token is drawn
  int32_t trow;      // packed target row of p
  int32_t drow;      // k-1 of the draft row of q (residual)
  double lse_t;      // log2-sum-exp2 of target row times c
  double lse_d;      // same for the draft row
  double us;         // sampling uniform u'
  double pad;
};
static_assert(sizeof(Job) == 48, "job size");

__host__ __device__ inline int esize_of(int dtype) { return dtype == DSP_BF16 ? 2 : 4; }

// Chunks per row so that one chunk is at most kChunkVecs 16-byte vectors.
__host__ __device__ inline int stat_chunks(int V, int esize) {
  const long pv = 16 / esize;
  const long nvec = (V + pv - 1) / pv;
  const long n = (nvec + kChunkVecs - 1) / kChunkVecs;
  return n < 1 ? 1 : (int)n;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static float val(const uint16_t* p, long i) { return bf16_val(p[i]); }
  __device__ static void unpack(u32x4 w, float* x) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = bf16_lo(w[q]);
      x[2 * q + 1] = bf16_hi(w[q]);
    }
  }
};
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ static float val(const float* p, long i) { return p[i]; }
  __device__ static void unpack(u32x4 w, float* x) {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(w[q]);
  }
};

// Row split: [0, head) scalar, [head, tail) as 16-byte vectors, [tail, V) scalar.
struct RowGeom {
  int head, nvec, tail;
};
template <typename T> __device__ __forceinline__ RowGeom row_geom(const T* p, int V) {
  constexpr int PV = Elem<T>::kPerVec;
  const uintptr_t a = (uintptr_t)p;
  int head = (int)(((16u - (uint32_t)(a & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const int nvec = (V - head) / PV;
  return {head, nvec, head + nvec * PV};
}

// Partial log2-sum-exp2 of a set of logits times c: the set's sum of 2^(x c - ref),
// with ref the set's maximum times c (-inf and 0 for an empty set).
struct LsePart {
  float ref;
  float pad;
  double sum;
};

// Merge of two partials: factors 2^(ref - max) <= 1 in fp32, products and sum in fp64.
// Symmetric bit for bit (fp contraction is off), so both lanes of a butterfly pair end
// with the same value.
__device__ __forceinline__ void lse_merge(float& r, double& s, float r2, double s2) {
  const float H = fmaxf(r, r2);
  if (H != -INFINITY) {
    const double a = s * (double)fast_exp2(r - H);
    const double b = s2 * (double)fast_exp2(r2 - H);
    s = a + b;
  }
  r = H;
}
// Sum over the wavefront by xor butterflies; fp64 addition commutes, so every lane ends
// with the same bits.
template <int TS> __device__ __forceinline__ double sum_xor_step(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = xor_lane<TS>((uint32_t)b), hi = xor_lane<TS>((uint32_t)(b >> 32));
  return v + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_xor(double s) {
  s = sum_xor_step<1>(s);
  s = sum_xor_step<2>(s);
  s = sum_xor_step<4>(s);
  s = sum_xor_step<8>(s);
  s = sum_xor_step<16>(s);
  return sum_xor_step<32>(s);
}
template <int TS> __device__ __forceinline__ float max_xor_step(float v) {
  return fmaxf(v, __uint_as_float(xor_lane<TS>(__float_as_uint(v))));
}

// One (row, chunk) of the sampled statistics pass: the wavefront's maximum is the
// reference of all its lanes' exp2 sums, which are then added by butterflies, and one
// LDS exchange merges the wavefronts (double-buffered by *phase, so a workgroup that
// loops over items needs a single barrier per item).
// The slot is written only if chk is null or *chk == chk_val (read after the row's
// loads are issued, so its latency overlaps them); returns whether it was.
template <typename T>
__device__ __forceinline__ bool chunk_stats(const T* __restrict__ row, int V, int nch, int c,
                                            float cl, StatSlot* __restrict__ out,
                                            LsePart (*sml)[kThreads / 64], int* phase,
                                            const int32_t* chk = nullptr, int chk_val = 0) {
  constexpr int PV = Elem<T>::kPerVec;
  const RowGeom g = row_geom(row, V);
  const int cv = (g.nvec + nch - 1) / nch;
  const int v0 = c * cv;
  const int v1 = min(g.nvec, v0 + cv);
  const u32x4* vp = (const u32x4*)(row + g.head);
  const int tid = threadIdx.x;

  int chk_got = chk ? *chk : chk_val;
  u32x4 buf[kVpt];
#pragma unroll
  for (int j = 0; j < kVpt; ++j) {
    const int v = v0 + tid + j * kThreads;
    if (v < v1) buf[j] = __builtin_nontemporal_load(vp + v);
  }
  // this thread's scalar elements: one of the unaligned head, one of the tail
  float sh = -INFINITY, st = -INFINITY;
  if (c == 0 && tid < g.head) sh = Elem<T>::val(row, tid);
  if (c == nch - 1 && tid < V - g.tail) st = Elem<T>::val(row, g.tail + tid);
  asm volatile("" : "+v"(chk_got));  // the check lands here, while the row is in flight
  const bool ok = chk_got == chk_val;

  float m = fmaxf(sh, st);
#pragma unroll
  for (int j = 0; j < kVpt; ++j) {
    const int v = v0 + tid + j * kThreads;
    if (v < v1) {
      float x[PV];
      Elem<T>::unpack(buf[j], x);
#pragma unroll
      for (int e = 0; e < PV; ++e) m = fmaxf(m, x[e]);
    }
  }
  // the exp pass converts the raw vectors again: keeping 8 fp32 values per vector live
  // instead would cost registers and therefore occupancy
#pragma unroll
  for (int j = 0; j < kVpt; ++j) asm volatile("" : "+v"(buf[j]));
  // one reference per wavefront (its maximum), so the lane sums need no rescaling
  m = max_xor_step<1>(m);
  m = max_xor_step<2>(m);
  m = max_xor_step<4>(m);
  m = max_xor_step<8>(m);
  m = max_xor_step<16>(m);
  m = max_xor_step<32>(m);
  float ref = m * cl;
  double s = 0.0;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kVpt; ++j) {
      const int v = v0 + tid + j * kThreads;
      if (v < v1) {
        float e8[PV];
        float x[PV];
        Elem<T>::unpack(buf[j], x);
#pragma unroll
        for (int e = 0; e < PV; ++e) e8[e] = fast_exp2(__builtin_fmaf(x[e], cl, -ref));
        // pairwise within the vector, fp64 across vectors
#pragma unroll
        for (int w = PV / 2; w > 0; w >>= 1)
#pragma unroll
          for (int e = 0; e < w; ++e) e8[e] += e8[e + w];
        s += (double)e8[0];
      }
    }
    if (sh != -INFINITY) s += (double)fast_exp2(__builtin_fmaf(sh, cl, -ref));
    if (st != -INFINITY) s += (double)fast_exp2(__builtin_fmaf(st, cl, -ref));
  }
  s = wave_sum_xor(s);
  LsePart* buf2 = sml[*phase];
  *phase ^= 1;
  if ((tid & 63) == 0) buf2[tid >> 6] = LsePart{ref, 0.f, s};
  __syncthreads();
  if (!ok) return false;
  if (tid == 0) {
    float R = buf2[0].ref;
    double S = buf2[0].sum;
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) lse_merge(R, S, buf2[w].ref, buf2[w].sum);
    out->ref = R;
    out->flag = (R == INFINITY || R != R) ? 1u : 0u;
    out->sum = S;
  }
  return true;
}

// One (row, chunk) of the greedy pass: (max value, lowest index) as a 64-bit key.
template <typename T>
__device__ __forceinline__ void chunk_argmax(const T* __restrict__ row, int V, int nch, int c,
                                             uint64_t* __restrict__ out, uint64_t* smk) {
  constexpr int PV = Elem<T>::kPerVec;
  const RowGeom g = row_geom(row, V);
  const int cv = (g.nvec + nch - 1) / nch;
  const int v0 = c * cv;
  const int v1 = min(g.nvec, v0 + cv);
  const u32x4* vp = (const u32x4*)(row + g.head);
  const int tid = threadIdx.x;

  u32x4 buf[kVpt];
#pragma unroll
  for (int j = 0; j < kVpt; ++j) {
    const int v = v0 + tid + j * kThreads;
    if (v < v1) buf[j] = __builtin_nontemporal_load(vp + v);
  }
  float best = -INFINITY;
  int bidx = -1;
  if (c == 0 && tid < g.head) {
    best = Elem<T>::val(row, tid);
    bidx = tid;
  }
  // visit in increasing token order; strict '>' keeps the lowest index of equal values
#pragma unroll
  for (int j = 0; j < kVpt; ++j) {
    const int v = v0 + tid + j * kThreads;
    if (v < v1) {
      float x[PV];
      Elem<T>::unpack(buf[j], x);
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        const bool gt = x[e] > best || bidx < 0;
        best = gt ? x[e] : best;
        bidx = gt ? g.head + v * PV + e : bidx;
      }
    }
  }
  if (c == nch - 1 && tid < V - g.tail) {
    const float x = Elem<T>::val(row, g.tail + tid);
    if (x > best || bidx < 0) {
      best = x;
      bidx = g.tail + tid;
    }
  }
  const uint64_t key = bidx < 0 ? 0ull : amax_key(best, (uint32_t)bidx);
  const uint64_t K = block_max<kThreads / 64>(key, smk);
  if (tid == 0) *out = K;
}

struct StatsArgs {
  const void* tgt;
  int64_t ld_t;
  const void* drf;
  int64_t ld_d_r, ld_d_k;
  const int32_t* cu;
  int32_t R, K, V, max_rows;
  int32_t ncht, nchd;
  float cl;
  StatSlot* tstats;
  StatSlot* dstats;
  uint64_t* round_dev;  // sampled path: advanced once per call here, read by the decisions
  const int32_t* row_req;  // optional packed-row maps (request, position) from the ragged pack
  const int32_t* row_pos;
};

template <typename TT>
__global__ __launch_bounds__(kThreads) void verify_argmax_kernel(StatsArgs a) {
  __shared__ uint64_t smk[kThreads / 64];
  const int tot = a.cu[a.R];
  const int T_rows = tot < 0 ? 0 : (tot > a.max_rows ? a.max_rows : tot);
  const long items = (long)T_rows * a.ncht;
  uint64_t* keys = (uint64_t*)a.tstats;
  for (long it = blockIdx.x; it < items; it += gridDim.x) {
    const int row = (int)(it / a.ncht), c = (int)(it % a.ncht);
    const TT* p = (const TT*)a.tgt + (size_t)row * a.ld_t;
    chunk_argmax<TT>(p, a.V, a.ncht, c, keys + 2 * it, smk);
  }
}

// log2-sum-exp2 of a row from its chunk slots (fp64). Sets *bad for non-finite rows.
__device__ __forceinline__ double merge_lse(const StatSlot* s, int nch, bool* bad) {
  // slots are read 16 at a time, all loads issued before any is used (one memory
  // latency per batch instead of one per chunk), then merged online in fp64. The
  // loads are unconditional (slots past the row repeat its last one and are masked
  // after): a load under a branch makes the compiler wait for it on the spot.
  constexpr int B = 16;
  float H = -INFINITY;
  double S = 0.0;
  bool f = false;
  for (int c0 = 0; c0 < nch; c0 += B) {
    float ref[B];
    double sum[B];
    uint32_t flag[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const StatSlot v = s[c0 + q < nch ? c0 + q : nch - 1];
      const bool in = c0 + q < nch;
      ref[q] = in ? v.ref : -INFINITY;
      flag[q] = in ? v.flag : 0u;
      sum[q] = in ? v.sum : 0.0;
    }
    float Hb = H;
#pragma unroll
    for (int q = 0; q < B; ++q) {
      Hb = fmaxf(Hb, ref[q]);
      f |= flag[q] != 0u;
    }
    // chunk factors 2^(ref - max) <= 1 in fp32 (one v_exp_f32 each), products and sums in fp64
    double Sb = H == -INFINITY ? 0.0 : S * (double)fast_exp2(H - Hb);
#pragma unroll
    for (int q = 0; q < B; ++q)
      if (ref[q] != -INFINITY) Sb += sum[q] * (double)fast_exp2(ref[q] - Hb);
    H = Hb;
    S = Sb;
  }
  const double L = (double)H + log2(S);
  if (f || !(L == L) || L == INFINITY || L == -INFINITY) *bad = true;
  return L;
}

__device__ __forceinline__ uint32_t merge_argmax(const StatSlot* s, int nch) {
  const uint64_t* k = (const uint64_t*)s;
  constexpr int B = 16;
  uint64_t b = 0;
  for (int c0 = 0; c0 < nch; c0 += B) {
    uint64_t v[B];
#pragma unroll
    for (int q = 0; q < B; ++q) v[q] = c0 + q < nch ? k[2 * (c0 + q)] : 0ull;
#pragma unroll
    for (int q = 0; q < B; ++q) b = v[q] > b ? v[q] : b;
  }
  return amax_index(b);
}

template <typename T> __device__ __forceinline__ float load_elem(const void* base, size_t off) {
  return Elem<T>::val((const T*)base, (long)off);
}
struct DecideArgs {
  const void* tgt;
  int t_dtype;
  int64_t ld_t;
  const void* drf;
  int d_dtype;
  int64_t ld_d_r, ld_d_k;
  const int32_t* cu;
  const int32_t* x;
  int64_t ld_x;
  const int32_t* parent;
  int32_t R, K, V, max_rows;
  int32_t ncht, nchd;
  float cl;
  uint64_t seed, round;
  const int64_t* req_id;
  const StatSlot* tstats;
  const StatSlot* dstats;
  int32_t* acc_len;
  int32_t* out;
  int32_t* stop;
  float* p_x;
  float* q_x;
  int32_t* status;
  const uint64_t* round_dev;  // when set, the round is read from device memory
  const int32_t* cap;         // cap-accept commit windows (nullable)
  int32_t* ceiling;           // drafts accepted over the whole window (nullable)
};

// Cap-accept: the decisions cover the whole packed window n; only the first
// c = min(cap_i, n) positions are committed. Returns the committed stop position
// (first rejection if it lies inside the commit window, else c + 1, whose draw is
// then the bonus from p_{c+1}) and reports the full-window acceptance.
__device__ __forceinline__ int commit_stop(const DecideArgs& a, int i, int n, int kfull, int* cw) {
  int c = n;
  if (a.cap) {
    c = a.cap[i];
    c = c < 0 ? 0 : (c > n ? n : c);
  }
  *cw = c;
  if (a.ceiling && (threadIdx.x & 63) == 0) a.ceiling[i] = kfull - 1;
  return kfull <= c ? kfull : c + 1;
}

__device__ __forceinline__ float load_t(const DecideArgs& a, int row, int v) {
  const size_t off = (size_t)row * a.ld_t + v;
  return a.t_dtype == DSP_BF16 ? load_elem<uint16_t>(a.tgt, off) : load_elem<float>(a.tgt, off);
}
__device__ __forceinline__ float load_d(const DecideArgs& a, int i, int k0, int v) {
  const size_t off = (size_t)i * a.ld_d_r + (size_t)k0 * a.ld_d_k + v;
  return a.d_dtype == DSP_BF16 ? load_elem<uint16_t>(a.drf, off) : load_elem<float>(a.drf, off);
}

// Writes the all -1 fault record of request i (one wavefront).
__device__ void fault_request(const DecideArgs& a, int i, int bits) {
  const int lane = threadIdx.x & 63;
  for (int j = lane; j <= a.K; j += 64) a.out[(size_t)i * (a.K + 1) + j] = -1;
  if (a.p_x)
    for (int j = lane; j < a.K; j += 64) {
      a.p_x[(size_t)i * a.K + j] = 0.f;
      a.q_x[(size_t)i * a.K + j] = 0.f;
    }
  if (lane == 0) {
    a.acc_len[i] = -1;
    a.stop[i] = -1;
    atomicOr(a.status, bits);
  }
}

// Sampled decision of request i, run by one wavefront once all row statistics exist.
// The sampling job (residual at the first rejection, or the bonus row) goes to *jout.
template <typename TT, typename TD>
__device__ void decide_sampled(const DecideArgs& a, int i, Job* jout) {
  const int lane = threadIdx.x & 63;
  // Two rounds of memory latency: first everything addressed by (i, lane) alone (the
  // window, the draft tokens, the draft rows' statistics of every block position),
  // then what needs the packed base or the tokens (target statistics, the two logits).
  const int base = a.cu[i];
  const int nxt = a.cu[i + 1];
  const uint64_t rid = a.req_id ? (uint64_t)a.req_id[i] : (uint64_t)i;
  const uint64_t rnd = a.round_dev ? *a.round_dev : a.round;
  const int k = lane + 1;
  const bool blk = lane < a.K;
  int x = 0;
  if (blk) x = a.x[(size_t)i * a.ld_x + lane];
  // the uniforms need only the round and the request id: drawn while the statistics load
  uint64_t c[4] = {rnd, rid, (uint64_t)k, 0ull};
  philox4x64_10(c, a.seed, 0ull);
  const double u = unit_double(c[0]);
  const double us = unit_double(c[1]);
  bool bad_d = false;
  double lse_d = 0.0;  // slots past the window hold no statistics: used only for positions
  if (blk) lse_d = merge_lse(a.dstats + ((size_t)i * a.K + lane) * a.nchd, a.nchd, &bad_d);
  const int n = nxt - base - 1;
  const bool pos = k <= n;     // a draft position of the window
  const bool bon = lane == n;  // prepares the bonus row (n < 64)
  if (!pos) x = 0;
  const bool tokbad = pos && (x < 0 || x >= a.V);
  float tx = 0.f, dx = 0.f;
  if (pos && !tokbad) {
    tx = load_elem<TT>(a.tgt, (size_t)(base + lane) * a.ld_t + x);
    dx = load_elem<TD>(a.drf, (size_t)i * a.ld_d_r + (size_t)lane * a.ld_d_k + x);
  }
  bool bad = pos && bad_d;
  double lse_t = 0.0;
  if (pos || bon) lse_t = merge_lse(a.tstats + (size_t)(base + lane) * a.ncht, a.ncht, &bad);
  if (!pos) lse_d = 0.0;
  double lp2 = 0.0, lq2 = 0.0;
  bool acc = true;
  if (pos && !tokbad) {
    const double cl = (double)a.cl;
    lp2 = (double)tx * cl - lse_t;
    lq2 = (double)dx * cl - lse_d;
    acc = u < exp2(lp2 - lq2);
  }
  if (__ballot(tokbad)) {
    fault_request(a, i, DSP_STATUS_TOKEN_RANGE);
    if (lane == 0) jout->mode = JOB_NONE;
    return;
  }
  if (__ballot(pos && bad)) {
    fault_request(a, i, DSP_STATUS_NONFINITE);
    if (lane == 0) jout->mode = JOB_NONE;
    return;
  }
  const uint64_t rej = __ballot(pos && !acc);
  int cw;
  const int kstop = commit_stop(a, i, n, rej ? __ffsll((unsigned long long)rej) : n + 1, &cw);
  const int accepted = kstop - 1;
  if (a.p_x && lane < a.K) {
    a.p_x[(size_t)i * a.K + lane] = pos ? (float)exp2(lp2) : 0.f;
    a.q_x[(size_t)i * a.K + lane] = pos ? (float)exp2(lq2) : 0.f;
  }
  int32_t* orow = a.out + (size_t)i * (a.K + 1);
  if (lane < accepted) orow[lane] = x;
  else if (lane > accepted && lane <= a.K) orow[lane] = -1;
  if (a.K == 64 && lane == 0 && accepted < 64) orow[64] = -1;
  Job j;
  j.pad = 0.0;
  if (kstop <= cw) {
    if (k == kstop) {
      j.mode = JOB_RESID;
      j.kstop = kstop;
      j.trow = base + lane;
      j.drow = lane;
      j.lse_t = lse_t;
      j.lse_d = lse_d;
      j.us = us;
      *jout = j;
    }
  } else {
    // whole commit window accepted: bonus from the row after its last draft (lane cw
    // holds that row's statistics and the sampling uniform of position cw + 1)
    bool writer = cw < 64 ? lane == cw : lane == 0;
    if (writer) {
      double lt = lse_t, ub = us;
      bool b2 = bad;
      if (cw >= 64) {
        b2 = false;
        lt = merge_lse(a.tstats + (size_t)(base + cw) * a.ncht, a.ncht, &b2);
        uint64_t c2[4] = {rnd, rid, (uint64_t)(cw + 1), 0ull};
        philox4x64_10(c2, a.seed, 0ull);
        ub = unit_double(c2[1]);
      }
      j.mode = b2 ? JOB_NONE : JOB_BONUS;
      j.kstop = cw + 1;
      j.trow = base + cw;
      j.drow = -1;
      j.lse_t = lt;
      j.lse_d = 0.0;
      j.us = ub;
      *jout = j;
      if (b2) {
        orow[cw] = -1;
        atomicOr(a.status, DSP_STATUS_NONFINITE);
      }
    }
  }
  if (lane == 0) {
    a.acc_len[i] = accepted;
    a.stop[i] = kstop;
  }
}

// Request owning packed row p: largest i with cu[i] <= p (cu ascending).
__device__ __forceinline__ int find_request(const int32_t* cu, int R, int p) {
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

constexpr int kCuLds = 2048;  // requests whose offsets are staged in LDS for the row search

// Statistics pass (T > 0): every packed target row, and the draft row of every packed
// row that is not an anchor (so windows shorter than K cost no work). Items are numbered
// row by row, each row's target chunks before its draft chunks, so the items of rows at
// or past the device-side packed total form one tail: a workgroup stops at its first
// such item, and a grid capped below the item count (the caller's max_rows may be far
// above the packed total) costs no dispatch of idle workgroups past the cap. A draft
// item finds its (request, position) in the pack's row maps when the caller passes
// them, else by a binary search of cu_seqlens staged in LDS.
template <typename TT, typename TD>
__global__ __launch_bounds__(kThreads) void verify_stats_kernel(StatsArgs a, const int32_t* __restrict__ cu_,
                                                                 const int32_t* __restrict__ rq_,
                                                                 const int32_t* __restrict__ rp_) {
  // cu_seqlens and the row maps are only read here; as restrict-qualified parameters their
  // workgroup-uniform reads go through the scalar cache instead of one vector request per
  // wavefront to the same few lines
  __shared__ LsePart sml[2][kThreads / 64];
  __shared__ int32_t s_cu[kCuLds + 1];
  int phase = 0;
  if (a.round_dev && blockIdx.x == 0 && threadIdx.x == 0) *a.round_dev += 1;
  // an item's row and chunk follow from its number alone, so its metadata loads (the
  // packed total, the row maps) go out together, in one memory round trip
  const int nch = a.ncht + a.nchd;
  const int max_packed = (int)min((long)a.max_rows, (long)a.R * (a.K + 1));
  const long items = (long)max_packed * nch;
  bool staged = false;
  for (long it = blockIdx.x; it < items; it += gridDim.x) {
    const int row = (int)(it / nch), c = (int)(it % nch);
    if (c < a.ncht) {
      if (row >= cu_[a.R]) break;  // uniform over the workgroup; later items lie further on
      const TT* p = (const TT*)a.tgt + (size_t)row * a.ld_t;
      chunk_stats<TT>(p, a.V, a.ncht, c, a.cl, a.tstats + (size_t)row * a.ncht + c, sml, &phase);
      continue;
    }
    const int cd = c - a.ncht;
    if (rq_) {
      // the maps are read together with the packed total; their agreement with
      // cu_seqlens is checked while the row streams in, and a disagreeing pair falls
      // back to the search
      // (no branch between the three loads, so they are issued together)
      const int i = rq_[row];
      const int k0 = rp_[row] - 1;
      const int tot = cu_[a.R];
      asm volatile("" ::"v"(i), "v"(k0), "v"(tot));  // keep the three loads ahead of any branch
      const bool in_req = (i >= 0) & (i < a.R);
      const bool drafted = in_req & (k0 >= 0) & (k0 < a.K);
      if (row >= tot) break;
      if (drafted) {
        const TD* p = (const TD*)a.drf + (size_t)i * a.ld_d_r + (size_t)k0 * a.ld_d_k;
        if (chunk_stats<TD>(p, a.V, a.nchd, cd, a.cl, a.dstats + ((size_t)i * a.K + k0) * a.nchd + cd, sml,
                            &phase, cu_ + i, row - k0 - 1))
          continue;
      } else if (in_req && k0 == -1 && cu_[i] == row) {
        continue;  // anchor row: no draft logits
      }
      const int i2 = find_request(cu_, a.R, row);
      const int k2 = row - cu_[i2] - 1;
      if (k2 < 0 || k2 >= a.K) continue;
      const TD* p = (const TD*)a.drf + (size_t)i2 * a.ld_d_r + (size_t)k2 * a.ld_d_k;
      chunk_stats<TD>(p, a.V, a.nchd, cd, a.cl, a.dstats + ((size_t)i2 * a.K + k2) * a.nchd + cd, sml,
                      &phase);
      continue;
    }
    if (row >= cu_[a.R]) break;
    const bool cu_lds = a.R <= kCuLds;
    if (cu_lds && !staged) {
      for (int q = threadIdx.x; q <= a.R; q += kThreads) s_cu[q] = cu_[q];
      __syncthreads();
      staged = true;
    }
    const int32_t* cu = cu_lds ? s_cu : cu_;
    const int i = find_request(cu, a.R, row);
    const int k0 = row - cu[i] - 1;  // draft position - 1 (-1: the anchor row)
    if (k0 < 0 || k0 >= a.K) continue;  // uniform over the workgroup
    const TD* p = (const TD*)a.drf + (size_t)i * a.ld_d_r + (size_t)k0 * a.ld_d_k;
    chunk_stats<TD>(p, a.V, a.nchd, cd, a.cl, a.dstats + ((size_t)i * a.K + k0) * a.nchd + cd, sml,
                    &phase);
  }
}

// Chain decision, greedy (T == 0).
__global__ __launch_bounds__(64) void verify_decide_greedy(DecideArgs a) {
  const int i = blockIdx.x, lane = threadIdx.x;
  const int base = a.cu[i], end = a.cu[i + 1];
  const int n = end - base - 1;
  if (n < 0 || n > a.K || base < 0 || end > a.max_rows) {
    fault_request(a, i, DSP_STATUS_WINDOW_RANGE);
    return;
  }
  const int k = lane + 1;
  const bool active = k <= n;
  bool acc = true, tokbad = false;
  int x = -1, am = -1;
  if (active) {
    x = a.x[(size_t)i * a.ld_x + lane];
    tokbad = x < 0 || x >= a.V;
    am = (int)merge_argmax(a.tstats + (size_t)(base + lane) * a.ncht, a.ncht);
    acc = x == am;
  }
  if (__ballot(tokbad)) {
    fault_request(a, i, DSP_STATUS_TOKEN_RANGE);
    return;
  }
  const uint64_t rej = __ballot(active && !acc);
  int cw;
  const int kstop = commit_stop(a, i, n, rej ? __ffsll((unsigned long long)rej) : n + 1, &cw);
  const int accepted = kstop - 1;
  int32_t* orow = a.out + (size_t)i * (a.K + 1);
  if (lane < accepted) orow[lane] = x;
  else if (lane > accepted && lane <= a.K) orow[lane] = -1;
  if (a.K == 64 && lane == 0 && accepted < 64) orow[64] = -1;
  if (kstop <= cw) {
    if (k == kstop) orow[lane] = am;
  } else if (lane == 0) {
    orow[cw] = (int)merge_argmax(a.tstats + (size_t)(base + cw) * a.ncht, a.ncht);
  }
  if (a.p_x && lane < a.K) {
    a.p_x[(size_t)i * a.K + lane] = 0.f;
    a.q_x[(size_t)i * a.K + lane] = 0.f;
  }
  if (lane == 0) {
    a.acc_len[i] = accepted;
    a.stop[i] = kstop;
  }
}

// Greedy tree walk, one workgroup of kWalkThreads per request: from the root, the
// arg-max of the current node's target row (largest value, lowest token id) selects
// the child carrying that token, until no child does. Only the rows on the walked
// path are read -- at most D + 1 of the window's rows -- instead of every node's.
constexpr int kWalkThreads = 1024;
constexpr int kWalkVpt = 16;  // 16-byte vectors per thread per round

// Arg-max key (amax_key order) of row p over [0, V), all threads of the workgroup.
template <typename T>
__device__ uint64_t row_argmax_key(const T* __restrict__ p, int V, uint64_t* smk) {
  constexpr int PV = Elem<T>::kPerVec;
  const RowGeom g = row_geom(p, V);
  const u32x4* vp = (const u32x4*)(p + g.head);
  const int tid = threadIdx.x;
  uint64_t best = 0;
  if (tid < g.head) best = amax_key(Elem<T>::val(p, tid), (uint32_t)tid);
  if (tid < V - g.tail) {
    const uint64_t k = amax_key(Elem<T>::val(p, g.tail + tid), (uint32_t)(g.tail + tid));
    best = k > best ? k : best;
  }
  for (int v0 = tid; v0 < g.nvec; v0 += kWalkVpt * kWalkThreads) {
    u32x4 buf[kWalkVpt];
#pragma unroll
    for (int j = 0; j < kWalkVpt; ++j)  // every load issued first (clamped, masked after)
      buf[j] = __builtin_nontemporal_load(vp + min(v0 + j * kWalkThreads, g.nvec - 1));
#pragma unroll
    for (int j = 0; j < kWalkVpt; ++j) {
      const int v = v0 + j * kWalkThreads;
      if (v < g.nvec) {
        float x[PV];
        Elem<T>::unpack(buf[j], x);
#pragma unroll
        for (int e = 0; e < PV; ++e) {
          const uint64_t k = amax_key(x[e], (uint32_t)(g.head + v * PV + e));
          best = k > best ? k : best;
        }
      }
    }
  }
  return block_max<kWalkThreads / 64>(best, smk);
}

template <typename TT>
__global__ __launch_bounds__(kWalkThreads) void verify_tree_walk_kernel(DecideArgs a) {
  __shared__ uint64_t smk[kWalkThreads / 64];
  __shared__ int s_next, s_bad;
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int base = a.cu[i], end = a.cu[i + 1];
  const int nn = end - base - 1;
  if (nn < 0 || nn > a.K || base < 0 || end > a.max_rows) {  // uniform
    if (tid < 64) fault_request(a, i, DSP_STATUS_WINDOW_RANGE);
    return;
  }
  // the window's nodes, one per lane of the first wavefront
  int tok = -1, par = -2;
  if (tid < 64 && lane < nn) {
    tok = a.x[(size_t)i * a.ld_x + lane];
    par = a.parent[(size_t)i * a.ld_x + lane];
  }
  if (tid < 64) {
    const bool bad = __ballot(lane < nn && (tok < 0 || tok >= a.V)) != 0;
    if (lane == 0) s_bad = bad;
  }
  __syncthreads();
  if (s_bad) {  // uniform
    if (tid < 64) fault_request(a, i, DSP_STATUS_TOKEN_RANGE);
    return;
  }
  int32_t* orow = a.out + (size_t)i * (a.K + 1);
  int cur = -1, depth = 0, am = 0;
  while (true) {
    const TT* p = (const TT*)a.tgt + (size_t)(base + 1 + cur) * a.ld_t;
    am = (int)amax_index(row_argmax_key<TT>(p, a.V, smk));
    if (tid < 64) {
      const uint64_t m = __ballot(lane < nn && par == cur && tok == am);
      if (lane == 0) s_next = (m && depth < a.K) ? __ffsll((unsigned long long)m) - 1 : -1;
    }
    __syncthreads();
    const int j = s_next;
    __syncthreads();  // everyone has read s_next before the next level rewrites it
    if (j < 0) break;  // uniform
    if (tid == j) orow[depth] = tok;  // lane j of the first wavefront holds node j
    cur = j;
    ++depth;
  }
  for (int k = depth + 1 + tid; k <= a.K; k += kWalkThreads) orow[k] = -1;
  if (tid == 0) {
    orow[depth] = am;
    a.acc_len[i] = depth;
    a.stop[i] = cur;
  }
}

struct JobFrame {
  float t_hi, t_lo, d_hi, d_lo, cl;
  bool resid;
};
__device__ __forceinline__ JobFrame job_frame(const Job& j, float cl, bool resid) {
  JobFrame f;
  f.t_hi = (float)j.lse_t;
  f.t_lo = (float)(j.lse_t - (double)f.t_hi);
  f.d_hi = (float)j.lse_d;
  f.d_lo = (float)(j.lse_d - (double)f.d_hi);
  f.cl = cl;
  f.resid = resid;
  return f;
}
__device__ __forceinline__ float job_weight(const JobFrame& f, float t, float d) {
  const float p = fast_exp2(__builtin_fmaf(t, f.cl, -f.t_hi) - f.t_lo);
  if (!f.resid) return p;
  const float q = fast_exp2(__builtin_fmaf(d, f.cl, -f.d_hi) - f.d_lo);
  return fmaxf(p - q, 0.f);
}

template <typename T> __device__ __forceinline__ void load8(const T* p, bool vec, float* x) {
  if (vec) {
    if constexpr (sizeof(T) == 2) {
      const u32x4 w = *(const u32x4*)p;
      Elem<uint16_t>::unpack(w, x);
    } else {
      const u32x4 w0 = *(const u32x4*)p;
      const u32x4 w1 = *((const u32x4*)p + 1);
      Elem<float>::unpack(w0, x);
      Elem<float>::unpack(w1, x + 4);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = Elem<T>::val(p, e);
  }
}


// A bounded view of one logit row (base and extent made wave-uniform): a 16-byte
// load at a byte offset at or past the extent returns zeros and touches no memory,
// so loads can be issued unconditionally (no branch for the compiler to wait at).
constexpr uint32_t kRowOOB = 0x80000000u;  // past every extent (rows are under 2 GiB)
constexpr int kAuxNT = 2;                   // cache-policy operand of a buffer load: non-temporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Eight consecutive logits as raw 16-byte vectors (one for bf16, two for fp32).
template <typename T> struct Raw8 {
  u32x4 w[sizeof(T) / 2];
  // non-temporal: rows streamed once must not evict what the next
  // kernels of the step read (without the hint the scheduler and pack of the next step
  // measured 2-3 us slower)
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int q = 0; q < (int)(sizeof(T) / 2); ++q)
      w[q] = __builtin_amdgcn_raw_buffer_load_b128(r, off == kRowOOB ? kRowOOB : off + 16 * q, 0, kAuxNT);
  }
  __device__ __forceinline__ void unpack(float* x) const {
#pragma unroll
    for (int q = 0; q < (int)(sizeof(T) / 2); ++q) Elem<T>::unpack(w[q], x + q * Elem<T>::kPerVec);
  }
};

constexpr int kSampleThreads = 1024;
constexpr int kSampleGrain = kSampleThreads * 8;  // chunk granularity: one 8-element vector per sample thread

// Residual / bonus chunking: R * nch2 items of ce elements, ce = kSampleGrain (one
// 16-byte vector per thread of the draw, which then rescans its chunk in one round trip)
// unless a row would need more than 64 chunks, then the next multiple of it. Smaller
// chunks give more residual workgroups and a shorter rescan: at 256 requests and
// V = 151,936, 19 chunks of 8,192 take 9.3 + 7.9 us for the masses and the draw,
// 7 chunks of 24,576 took 12.2 + 10.5 us.
struct SampleGeom {
  int nch2, ce;
};
__host__ __device__ inline SampleGeom sample_geom(int V) {
  int n = (V + kSampleGrain - 1) / kSampleGrain;
  if (n > 64) n = 64;
  if (n < 1) n = 1;
  int ce = (V + n - 1) / n;
  ce = (ce + kSampleGrain - 1) / kSampleGrain * kSampleGrain;
  SampleGeom g;
  g.ce = ce;
  g.nch2 = (V + ce - 1) / ce;
  return g;
}

// Weights of 8 consecutive elements starting at e (16-byte loads when aligned, guarded tail).
template <typename TT, typename TD>
__device__ __forceinline__ float job_weight8(const JobFrame& f, const TT* tp, const TD* dp, bool t_al, bool d_al,
                                             int e, int V) {
  float t[8], d[8];
  float w = 0.f;
  if (e + 8 <= V) {
    load8<TT>(tp + e, t_al, t);
    if (f.resid) load8<TD>(dp + e, d_al, d);
#pragma unroll
    for (int q = 0; q < 8; ++q) w += job_weight(f, t[q], f.resid ? d[q] : 0.f);
  } else {
    for (int q = 0; e + q < V; ++q)
      w += job_weight(f, Elem<TT>::val(tp, e + q), f.resid ? Elem<TD>::val(dp, e + q) : 0.f);
  }
  return w;
}

// The weights of 8 consecutive elements starting at e (zero past V), one per element.
template <typename TT, typename TD>
__device__ __forceinline__ void job_weights8(const JobFrame& f, const TT* tp, const TD* dp, bool t_al, bool d_al,
                                             int e, int V, float* wv) {
  if (e + 8 <= V) {
    float t[8], d[8];
    load8<TT>(tp + e, t_al, t);
    if (f.resid) load8<TD>(dp + e, d_al, d);
#pragma unroll
    for (int q = 0; q < 8; ++q) wv[q] = job_weight(f, t[q], f.resid ? d[q] : 0.f);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      wv[q] = e + q < V ? job_weight(f, Elem<TT>::val(tp, e + q), f.resid ? Elem<TD>::val(dp, e + q) : 0.f)
                        : 0.f;
  }
}

// Sum of the job's weights over [e0, e0 + len) with 256 threads x 8 elements per step;
// up to kBatch steps of loads are issued before any is used.
template <typename TT, typename TD>
__device__ __forceinline__ double job_chunk_sum(const JobFrame& f, const TT* tp, const TD* dp, int e0, int len,
                                                int V) {
  constexpr int kBatch = (sizeof(TT) == 2 && sizeof(TD) == 2) ? 4 : 2;
  const bool t_al = (((uintptr_t)tp) & 15u) == 0;
  const bool d_al = !f.resid || (((uintptr_t)dp) & 15u) == 0;
  const int e1 = min(V, e0 + len);
  // unconditional bounded loads (a load under a branch is waited for on the spot)
  const __amdgpu_buffer_rsrc_t trs = row_rsrc(tp, (uint32_t)((size_t)V * sizeof(TT)));
  const __amdgpu_buffer_rsrc_t drs = row_rsrc(dp, f.resid ? (uint32_t)((size_t)V * sizeof(TD)) : 0u);
  double s = 0.0;
  for (int eb = e0 + threadIdx.x * 8; eb < e1; eb += kBatch * kThreads * 8) {
    Raw8<TT> rt[kBatch];
    Raw8<TD> rd[kBatch];
    bool fast[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = eb + b * kThreads * 8;
      fast[b] = e + 8 <= e1 && t_al && d_al;
      rt[b].load_buf(trs, fast[b] ? (uint32_t)(e * sizeof(TT)) : kRowOOB);
      rd[b].load_buf(drs, fast[b] && f.resid ? (uint32_t)(e * sizeof(TD)) : kRowOOB);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = eb + b * kThreads * 8;
      // the fast-path weights are computed unconditionally (an out-of-range vector read
      // zeros and is discarded by the select): a load used only under a branch is sunk
      // into it by the compiler, which then waits for it there
      float t[8], d[8];
      rt[b].unpack(t);
      rd[b].unpack(d);
      float wf = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) wf += job_weight(f, t[q], f.resid ? d[q] : 0.f);
      float w = fast[b] ? wf : 0.f;
      if (!fast[b] && e < e1) w = job_weight8<TT, TD>(f, tp, dp, false, false, e, e1);
      s += (double)w;
    }
  }
  return s;
}

// Decisions: one wavefront per request; writes the request's sampling job.
template <typename TT, typename TD>
__global__ __launch_bounds__(64) void verify_decide_kernel(DecideArgs a, Job* __restrict__ jobs) {
  const int i = blockIdx.x;
  const int base = a.cu[i], end = a.cu[i + 1];
  const int n = end - base - 1;
  if (n < 0 || n > a.K || base < 0 || end > a.max_rows) {
    fault_request(a, i, DSP_STATUS_WINDOW_RANGE);
    if (threadIdx.x == 0) jobs[i].mode = JOB_NONE;
    return;
  }
  decide_sampled<TT, TD>(a, i, jobs + i);
}

struct SampleArgs {
  const void* tgt;
  int64_t ld_t;
  const void* drf;
  int64_t ld_d_r, ld_d_k;
  int32_t R, K, V, nch2, ce;
  float cl;
  const Job* jobs;
  double* rsum;
  int32_t* out;
  const StatSlot* tstats;  // the statistics pass's target row slots
  int32_t ncht;
};

// Chunks of a draw: chunk c covers elements [begin(c), begin(c + 1)) of the row.
//   uniform (ce > 0): begin(c) = min(V, c * ce) -- the residual / streamed layout;
//   statistics (ce == 0): the statistics pass's chunks of the row, whose masses the
//   pass already summed: begin(0) = 0, begin(c) = head + min(nvec, c * cv) * PV for
//   0 < c < n, begin(n) = V (the unaligned head in chunk 0, the tail in the last).
struct DrawChunks {
  int n, ce, V, head, nvec, cv, pv;
  __device__ __forceinline__ int begin(int c) const {
    if (ce > 0) return min(V, c * ce);
    if (c <= 0) return 0;
    if (c >= n) return V;
    return head + min(nvec, c * cv) * pv;
  }
};
__device__ __forceinline__ DrawChunks uniform_chunks(const SampleArgs& a) {
  return DrawChunks{a.nch2, a.ce, a.V, 0, 0, 0, 0};
}
template <typename TT>
__device__ __forceinline__ DrawChunks stats_chunks(const SampleArgs& a, const TT* tp) {
  const RowGeom g = row_geom(tp, a.V);
  return DrawChunks{a.ncht, 0, a.V, g.head, g.nvec, (g.nvec + a.ncht - 1) / a.ncht, Elem<TT>::kPerVec};
}
// A bonus draw (from p) needs no pass over its row: p's mass in each statistics chunk is
// the chunk's sum of 2^(x c - ref) times 2^(ref - lse). Used while the row has at most 64
// chunks (the masses stay in one wavefront's lanes and the draw's 64-entry table).
__device__ __forceinline__ bool bonus_from_stats(const Job& jb, const SampleArgs& a) {
  return jb.mode == JOB_BONUS && a.ncht <= 64;
}
// lanes 0..63 of the first wavefront: the bonus row's per-chunk masses into s_csum
__device__ __forceinline__ void bonus_masses(const SampleArgs& a, const Job& jb, double* s_csum) {
  const int c = threadIdx.x;
  const StatSlot sl = a.tstats[(size_t)jb.trow * a.ncht + min(c, a.ncht - 1)];
  s_csum[c] = c < a.ncht && sl.ref != -INFINITY ? sl.sum * exp2((double)sl.ref - jb.lse_t) : 0.0;
}

// Residual / bonus weight sums per (request, chunk), grid-stride over items.
template <typename TT, typename TD>
__global__ __launch_bounds__(kThreads) void verify_residual_kernel(SampleArgs a) {
  __shared__ double smd[kThreads / 64];
  const long items = (long)a.R * a.nch2;
  for (long it = blockIdx.x; it < items; it += gridDim.x) {
    const int i = (int)(it / a.nch2), c = (int)(it % a.nch2);
    const Job jb = a.jobs[i];
    if (jb.mode == JOB_NONE || bonus_from_stats(jb, a)) continue;  // uniform over the workgroup
    const bool resid = jb.mode == JOB_RESID;
    const JobFrame f = job_frame(jb, a.cl, resid);
    const TT* tp = (const TT*)a.tgt + (size_t)jb.trow * a.ld_t;
    const TD* dp = resid ? (const TD*)a.drf + (size_t)i * a.ld_d_r + (size_t)jb.drow * a.ld_d_k : nullptr;
    const double S = block_sum<kThreads / 64>(job_chunk_sum<TT, TD>(f, tp, dp, c * a.ce, a.ce, a.V), smd);
    if (threadIdx.x == 0) a.rsum[it] = S;
  }
}

// Inverse-CDF draw of request i's job, one workgroup of NT threads: s_csum (LDS) holds
// the job's weight per chunk; locate the chunk holding u' * total, rescan it with
// contiguous per-thread ranges and an fp64 exclusive scan, and let the owning thread walk
// its range to the first element past the target. A thread's range is taken in batches
// of kDrawVecs vectors (8 elements each), one memory round trip per batch; a range of
// one batch keeps its weights in registers for the walk, a longer one is reloaded batch
// by batch by its owner.
constexpr int kDrawVecs = 4;
// The job's weights of the kDrawVecs vectors from element eb, masked to [.., r1): every
// load issued before any is used (bounded buffer loads; a vector past the range reads
// zeros and is masked, the row's ragged last vector takes the guarded element path).
template <typename TT, typename TD, int NV>
__device__ __forceinline__ void draw_batch(const JobFrame& f, const TT* tp, const TD* dp,
                                           __amdgpu_buffer_rsrc_t trs, __amdgpu_buffer_rsrc_t drs, bool al,
                                           int eb, int r1, float (&wv)[8 * NV]) {
  Raw8<TT> rt[NV];
  Raw8<TD> rd[NV];
  bool fast[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = eb + 8 * v;
    fast[v] = al && e + 8 <= r1;
    rt[v].load_buf(trs, fast[v] ? (uint32_t)(e * sizeof(TT)) : kRowOOB);
    rd[v].load_buf(drs, fast[v] && f.resid ? (uint32_t)(e * sizeof(TD)) : kRowOOB);
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = eb + 8 * v;
    float t[8], d[8];
    rt[v].unpack(t);
    rd[v].unpack(d);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float wq = job_weight(f, t[q], f.resid ? d[q] : 0.f);
      wv[8 * v + q] = fast[v] ? wq : 0.f;
    }
    if (!fast[v] && e < r1) {
      float w8[8];
      job_weights8<TT, TD>(f, tp, dp, false, false, e, r1, w8);
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[8 * v + q] = w8[q];
    }
  }
}

// The rescan of a draw's chunk: each thread's range [r0, r1) (per elements) summed in
// batches of NV vectors, an fp64 exclusive scan over the workgroup, and the walk of the
// range holding tau by its owner, which records the first element past it in *found.
template <typename TT, typename TD, int NV, int NW>
__device__ __forceinline__ void draw_rescan(const JobFrame& f, const TT* tp, const TD* dp,
                                            __amdgpu_buffer_rsrc_t trs, __amdgpu_buffer_rsrc_t drs, bool al,
                                            int r0, int r1, int per, double tau, double* s_wtot, int* found) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int BE = 8 * NV;  // elements per batch
  const int nb = (per + BE - 1) / BE;  // batches per thread (uniform)
  float wv[BE];
  double s = 0.0;
  for (int b = 0; b < nb; ++b) {
    draw_batch<TT, TD, NV>(f, tp, dp, trs, drs, al, r0 + b * BE, r1, wv);
#pragma unroll
    for (int q = 0; q < BE; ++q) s += (double)wv[q];
  }
  double inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_wtot[w] = inc;
  __syncthreads();
  double off = 0.0;
  for (int q = 0; q < w; ++q) off += s_wtot[q];
  const double E = off + inc - s;
  if (E <= tau && tau < E + s) {
    // the owner walks its range again batch by batch (a single batch is still in registers)
    double run = E;
    int hit = -1;
    for (int b = 0; b < nb && hit < 0; ++b) {
      if (nb > 1) draw_batch<TT, TD, NV>(f, tp, dp, trs, drs, al, r0 + b * BE, r1, wv);
#pragma unroll
      for (int q = 0; q < BE; ++q) {
        run += (double)wv[q];
        if (hit < 0 && r0 + b * BE + q < r1 && run > tau) hit = r0 + b * BE + q;
      }
    }
    if (hit >= 0) atomicMin(found, hit);
  }
}

template <typename TT, typename TD, int NT>
__device__ void sample_draw(const SampleArgs& a, int i, const Job& jb, double* s_csum, const DrawChunks& dc) {
  constexpr int NW = NT / 64;
  constexpr int kGrain = NT * 8;
  __shared__ double s_wtot[NW];
  __shared__ int s_chunk;
  __shared__ double s_tau;
  __shared__ int s_found;
  __shared__ int s_lastp[NW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  bool resid = jb.mode == JOB_RESID;
  const TT* tp = (const TT*)a.tgt + (size_t)jb.trow * a.ld_t;
  const TD* dp = resid ? (const TD*)a.drf + (size_t)i * a.ld_d_r + (size_t)jb.drow * a.ld_d_k : nullptr;
  double total = 0.0;
  for (int c = 0; c < dc.n; ++c) total += s_csum[c];
  if (resid && !(total > 0.0)) {
    // empty residual (p <= q everywhere after rounding): draw from p instead
    resid = false;
    const JobFrame fp = job_frame(jb, a.cl, false);
    for (int c = 0; c < dc.n; ++c) {
      double s0 = 0.0;
      const int c0 = dc.begin(c), c1 = dc.begin(c + 1);
      const bool t_al0 = (((uintptr_t)(tp + c0)) & 15u) == 0;
      for (int e = c0 + tid * 8; e < c1; e += NT * 8)
        s0 += (double)job_weight8<TT, TD>(fp, tp, nullptr, t_al0, true, e, c1);
      const double S = block_sum<NW>(s0, s_wtot);
      __syncthreads();
      if (tid == 0) s_csum[c] = S;
      __syncthreads();
    }
    total = 0.0;
    for (int c = 0; c < dc.n; ++c) total += s_csum[c];
  }
  const JobFrame f = job_frame(jb, a.cl, resid);
  if (tid == 0) {
    const double target = jb.us * total;
    double acc = 0.0;
    int cs = -1;
    for (int c = 0; c < dc.n; ++c) {
      if (acc + s_csum[c] > target) {
        cs = c;
        break;
      }
      acc += s_csum[c];
    }
    double tau = target - acc;
    if (cs < 0) {  // rounding left no chunk: take the last chunk with weight
      for (int c = dc.n - 1; c >= 0; --c)
        if (s_csum[c] > 0.0) {
          cs = c;
          break;
        }
      tau = INFINITY;
    }
    s_chunk = cs;
    s_tau = tau;
    s_found = 0x7fffffff;
  }
  __syncthreads();
  const int cs = s_chunk;
  const double tau = s_tau;
  int32_t* dst = a.out + (size_t)i * (a.K + 1) + jb.kstop - 1;
  if (cs < 0) {
    if (tid == 0) *dst = -1;
    return;
  }
  const int e0 = dc.begin(cs), e1 = dc.begin(cs + 1);
  // contiguous per-thread ranges, a multiple of 8 elements each
  const int per = (e1 - e0 + kGrain - 1) / kGrain * 8;
  const int r0 = min(e1, e0 + tid * per), r1 = min(e1, r0 + per);
  // vector loads need 16-byte aligned ranges: the uniform chunks start at multiples of 8
  // elements; a statistics chunk of an unaligned row may not
  const bool t_al = (((uintptr_t)(tp + e0)) & 15u) == 0 && (e0 % 8) == 0;
  const bool d_al = !resid || ((((uintptr_t)dp) & 15u) == 0 && (e0 % 8) == 0);
  // the range in batches of kDrawVecs vectors, each batch's loads issued together
  const __amdgpu_buffer_rsrc_t trs = row_rsrc(tp, (uint32_t)((size_t)a.V * sizeof(TT)));
  const __amdgpu_buffer_rsrc_t drs = row_rsrc(dp, resid ? (uint32_t)((size_t)a.V * sizeof(TD)) : 0u);
  // batches as long as the range, up to kDrawVecs vectors (unused vectors measured
  // slower on short ranges)
  const int nv = min(kDrawVecs, max(1, per / 8));  // uniform
  const bool al = t_al && d_al;
  if (nv == 1) draw_rescan<TT, TD, 1, NW>(f, tp, dp, trs, drs, al, r0, r1, per, tau, s_wtot, &s_found);
  else if (nv == 2) draw_rescan<TT, TD, 2, NW>(f, tp, dp, trs, drs, al, r0, r1, per, tau, s_wtot, &s_found);
  else if (nv == 3) draw_rescan<TT, TD, 3, NW>(f, tp, dp, trs, drs, al, r0, r1, per, tau, s_wtot, &s_found);
  else draw_rescan<TT, TD, 4, NW>(f, tp, dp, trs, drs, al, r0, r1, per, tau, s_wtot, &s_found);
  __syncthreads();
  if (s_found == 0x7fffffff) {
    // rounding put the target past the rescanned total: last token with weight in the chunk
    int last_pos = -1;
    for (int e = r1 - 1; e >= r0 && last_pos < 0; --e)
      if (job_weight(f, Elem<TT>::val(tp, e), resid ? Elem<TD>::val(dp, e) : 0.f) > 0.f) last_pos = e;
    const int lp = block_max<NW>(last_pos, s_lastp);
    if (tid == 0) s_found = lp;
    __syncthreads();
  }
  if (tid == 0) *dst = s_found;
}

template <typename TT, typename TD>
__global__ __launch_bounds__(kSampleThreads) void verify_sample_kernel(SampleArgs a) {
  __shared__ double s_csum[64];
  const int i = blockIdx.x, tid = threadIdx.x;
  const Job jb = a.jobs[i];
  if (jb.mode == JOB_NONE) return;
  const bool st = bonus_from_stats(jb, a);
  if (tid < 64) {
    if (st) bonus_masses(a, jb, s_csum);
    else s_csum[tid] = tid < a.nch2 ? a.rsum[(size_t)i * a.nch2 + tid] : 0.0;
  }
  __syncthreads();
  const TT* tp = (const TT*)a.tgt + (size_t)jb.trow * a.ld_t;
  sample_draw<TT, TD, kSampleThreads>(a, i, jb, s_csum, st ? stats_chunks<TT>(a, tp) : uniform_chunks(a));
}

struct VerifyLayout {
  int ncht, nchd, max_rows;
  SampleGeom sg;
  size_t off_t, off_d, off_j, off_r, total;
};

VerifyLayout verify_layout(int R, int K, int V, int max_rows, int t_dtype, int d_dtype) {
  VerifyLayout L;
  L.max_rows = max_rows > 0 ? max_rows : R * (K + 1);
  L.ncht = stat_chunks(V, esize_of(t_dtype));
  L.nchd = stat_chunks(V, esize_of(d_dtype));
  L.sg = sample_geom(V);
  size_t off = 0;
  L.off_t = off;
  off = align_up(off + (size_t)L.max_rows * L.ncht * sizeof(StatSlot), 256);
  L.off_d = off;
  off = align_up(off + (size_t)R * K * L.nchd * sizeof(StatSlot), 256);
  L.off_j = off;
  off = align_up(off + (size_t)R * sizeof(Job), 256);
  L.off_r = off;
  off = align_up(off + (size_t)R * L.sg.nch2 * sizeof(double), 256);
  L.total = off;
  return L;
}

// Workgroups of the statistics pass. Up to kStatsOneEach items, one item each: when
// every item is live that is the fastest shape (measured: a workgroup looping over ~10
// items costs ~8% on the 256 x 16 full-window run). Larger launches get kStatsGridCap
// workgroups that loop: max_rows is then often far above the device-side packed total
// (one graph captured for the largest batch), and a workgroup left without a live item
// still costs its dispatch (~0.7 ns each: 98 us instead of 37 for 472 live rows under
// max_rows = 4,352 at V = 151,936).
constexpr long kStatsOneEach = 16384;
constexpr long kStatsGridCap = 8192;
long stats_grid(long max_items) {
  long g = max_items <= kStatsOneEach ? max_items : kStatsGridCap;
  return g < 1 ? 1 : g;
}

template <typename TT, typename TD>
void launch_sampled(const StatsArgs& sa, const DecideArgs& da, const SampleArgs& pa, hipStream_t s,
                    long max_items) {
  const long g = stats_grid(max_items);
  launch(DSP_K_VERIFY_STATS, verify_stats_kernel<TT, TD>, dim3((unsigned)g), dim3(kThreads), 0, s, sa, sa.cu,
         sa.row_req, sa.row_pos);
  // decisions, then the residual / bonus masses spread over every CU (one workgroup per
  // (request, chunk) item: most items belong to bonus jobs, whose masses the statistics
  // pass holds, and exit at once, so a grid-stride loop would only chain their job loads
  // one after another), then one draw per request. (One workgroup per request doing all
  // three measured slower even with a request for nearly every CU: 36.6 against 31 us at
  // 256 requests, V = 151,936.)
  launch(DSP_K_VERIFY_DECIDE, verify_decide_kernel<TT, TD>, dim3(da.R), dim3(64), 0, s, da, (Job*)pa.jobs);
  const long ri = (long)pa.R * pa.nch2;
  const long g2 = ri < (1l << 20) ? ri : (1l << 20);
  launch(DSP_K_VERIFY_RESIDUAL, verify_residual_kernel<TT, TD>, dim3((unsigned)g2), dim3(kThreads), 0, s, pa);
  launch(DSP_K_VERIFY_SAMPLE, verify_sample_kernel<TT, TD>, dim3(pa.R), dim3(kSampleThreads), 0, s, pa);
}

template <typename TT>
void launch_greedy(const StatsArgs& sa, const DecideArgs& da, hipStream_t s, long max_items, bool tree) {
  if (tree) {
    launch(DSP_K_VERIFY_DECIDE, verify_tree_walk_kernel<TT>, dim3(da.R), dim3(kWalkThreads), 0, s, da);
    return;
  }
  const long g = stats_grid(max_items);
  launch(DSP_K_VERIFY_STATS, verify_argmax_kernel<TT>, dim3((unsigned)g), dim3(kThreads), 0, s, sa);
  launch(DSP_K_VERIFY_DECIDE, verify_decide_greedy, dim3(da.R), dim3(64), 0, s,
         da);
}

}  // namespace
}  // namespace dsp
using namespace dsp;

extern "C" size_t dsp_verify_rejection_workspace_size(int32_t R, int32_t K, int32_t V, int32_t max_rows,
                                                      int32_t t_dtype, int32_t d_dtype) {
  if (R < 1 || K < 1 || V < 1 || max_rows < 0) return 0;
  return verify_layout(R, K, V, max_rows, t_dtype, d_dtype).total;
}

// The allocation-free entry point's scratch: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends. Its size bounds the batches that
// entry point accepts. Host code never uses the array's name as an address (on the host
// it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int32_t scratch_address(void** out) {
  int dev = -1;
  const hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return hip_check(e0, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DSP_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_check(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DSP_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSP_OK;
}
}  // namespace

// Shared by both verify entry points: with noalloc the workspace is the current device's
// `scratch` (ws and ws_bytes are ignored), after the arguments have been checked.
static int32_t verify_impl(const void* tgt, int32_t t_dtype, int64_t ld_t, const int32_t* cu_seqlens,
                           const void* drf, int32_t d_dtype, int64_t ld_d_r, int64_t ld_d_k,
                           const int32_t* draft_tok, int64_t ld_x, const int32_t* parent, int32_t R, int32_t K,
                           int32_t V, int32_t max_rows, float temperature, uint64_t seed, uint64_t round,
                           uint64_t* round_dev, const int64_t* req_id, const int32_t* row_req,
                           const int32_t* row_pos, const int32_t* cap, int32_t* ceiling, int32_t* accepted_len,
                           int32_t* out_tokens, int32_t* stop_pos, float* p_x, float* q_x, int32_t* status,
                           void* ws, size_t ws_bytes, bool noalloc, void* stream) {
  clear_error();
  if (R < 1 || K < 1 || K > 64 || V < 1)
    return fail(DSP_ERR_SHAPE, "need R >= 1, 1 <= K <= 64, V >= 1 (R=%d K=%d V=%d)", R, K, V);
  if (t_dtype != DSP_F32 && t_dtype != DSP_BF16) return fail(DSP_ERR_DTYPE, "bad target dtype %d", t_dtype);
  if ((int64_t)V * 4 >= ((int64_t)1 << 31)) return fail(DSP_ERR_SHAPE, "V too large: rows must stay under 2 GiB");
  if (!(temperature >= 0.f) || temperature == INFINITY)
    return fail(DSP_ERR_SHAPE, "temperature must be finite and >= 0");
  const bool greedy = temperature == 0.f;
  const bool tree = parent != nullptr;
  if (tree && (cap || ceiling)) return fail(DSP_ERR_UNSUPPORTED, "cap-accept applies to chain verify only");
  if (tree && !greedy) return fail(DSP_ERR_UNSUPPORTED, "tree verify supports temperature 0 only");
  if (!greedy && d_dtype != DSP_F32 && d_dtype != DSP_BF16)
    return fail(DSP_ERR_DTYPE, "bad draft dtype %d", d_dtype);
  if (!tgt || !cu_seqlens || !draft_tok || !accepted_len || !out_tokens || !stop_pos || !status)
    return fail(DSP_ERR_NULL, "required pointer is NULL");
  if (!greedy && !drf) return fail(DSP_ERR_NULL, "draft logits required for temperature > 0");
  if ((p_x == nullptr) != (q_x == nullptr)) return fail(DSP_ERR_NULL, "p_x and q_x go together");
  if ((row_req == nullptr) != (row_pos == nullptr)) return fail(DSP_ERR_NULL, "row_req and row_pos go together");
  if (ld_t < V || ld_x < K) return fail(DSP_ERR_SHAPE, "strides too small");
  if (!greedy && (ld_d_k < V || ld_d_r < (int64_t)K * ld_d_k))
    return fail(DSP_ERR_SHAPE, "draft strides too small");
  if (max_rows < 0 || max_rows > R * (K + 1)) return fail(DSP_ERR_SHAPE, "max_rows out of range");
  if (((uintptr_t)tgt) % esize_of(t_dtype) || (!greedy && ((uintptr_t)drf) % esize_of(d_dtype)))
    return fail(DSP_ERR_ALIGN, "logits must be aligned to their element size");
  const int ddt = greedy ? DSP_BF16 : d_dtype;
  const VerifyLayout L = verify_layout(R, K, V, max_rows, t_dtype, ddt);
  if (noalloc) {
    if (L.total > kNoAllocScratchBytes)
      return fail(DSP_ERR_WORKSPACE,
                  "this batch needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                  "(use dsp_verify_rejection with a workspace)", L.total, kNoAllocScratchBytes);
    const int32_t rc = scratch_address(&ws);
    if (rc != DSP_OK) return rc;
    ws_bytes = kNoAllocScratchBytes;
  }
  if (!ws || ws_bytes < L.total) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);

  StatSlot* tstats = (StatSlot*)((uintptr_t)ws + L.off_t);
  StatSlot* dstats = (StatSlot*)((uintptr_t)ws + L.off_d);
  Job* jobs = (Job*)((uintptr_t)ws + L.off_j);
  double* rsum = (double*)((uintptr_t)ws + L.off_r);
  const float cl = greedy ? 0.f : (float)(1.4426950408889634074 / (double)temperature);
  hipStream_t s = (hipStream_t)stream;

  StatsArgs sa{tgt, ld_t, drf, ld_d_r, ld_d_k, cu_seqlens, R, K, V, L.max_rows, L.ncht, L.nchd, cl,
               tstats, dstats, greedy ? nullptr : round_dev, row_req, row_pos};
  DecideArgs da{tgt, t_dtype, ld_t, drf, ddt, ld_d_r, ld_d_k, cu_seqlens, draft_tok, ld_x, parent,
                R, K, V, L.max_rows, L.ncht, L.nchd, cl, seed, round, req_id, tstats, dstats,
                accepted_len, out_tokens, stop_pos, p_x, q_x, status, round_dev, cap, ceiling};
  if (greedy) {
    const long max_items = (long)L.max_rows * L.ncht;
    if (t_dtype == DSP_BF16) launch_greedy<uint16_t>(sa, da, s, max_items, tree);
    else launch_greedy<float>(sa, da, s, max_items, tree);
  } else {
    SampleArgs pa{tgt, ld_t, drf, ld_d_r, ld_d_k, R, K, V, L.sg.nch2, L.sg.ce, cl, jobs, rsum, out_tokens,
                  tstats, L.ncht};
    const long max_items = (long)L.max_rows * (L.ncht + L.nchd);
    if (t_dtype == DSP_BF16 && d_dtype == DSP_BF16) launch_sampled<uint16_t, uint16_t>(sa, da, pa, s, max_items);
    else if (t_dtype == DSP_BF16) launch_sampled<uint16_t, float>(sa, da, pa, s, max_items);
    else if (d_dtype == DSP_BF16) launch_sampled<float, uint16_t>(sa, da, pa, s, max_items);
    else launch_sampled<float, float>(sa, da, pa, s, max_items);
  }
  return hip_check(hipGetLastError(), "verify launch");
}

extern "C" int32_t dsp_verify_rejection(const void* tgt, int32_t t_dtype, int64_t ld_t,
                                        const int32_t* cu_seqlens, const void* drf, int32_t d_dtype,
                                        int64_t ld_d_r, int64_t ld_d_k, const int32_t* draft_tok,
                                        int64_t ld_x, const int32_t* parent, int32_t R, int32_t K,
                                        int32_t V, int32_t max_rows, float temperature, uint64_t seed,
                                        uint64_t round, uint64_t* round_dev, const int64_t* req_id,
                                        const int32_t* row_req, const int32_t* row_pos,
                                        const int32_t* cap, int32_t* ceiling, int32_t* accepted_len,
                                        int32_t* out_tokens, int32_t* stop_pos, float* p_x, float* q_x,
                                        int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  return verify_impl(tgt, t_dtype, ld_t, cu_seqlens, drf, d_dtype, ld_d_r, ld_d_k, draft_tok, ld_x, parent, R, K,
                     V, max_rows, temperature, seed, round, round_dev, req_id, row_req, row_pos, cap, ceiling,
                     accepted_len, out_tokens, stop_pos, p_x, q_x, status, ws, ws_bytes, false, stream);
}

extern "C" int32_t dsp_verify_rejection_noalloc(const void* tgt, int32_t t_dtype, int64_t ld_t,
                                                const int32_t* cu_seqlens, const void* drf, int32_t d_dtype,
                                                int64_t ld_d_r, int64_t ld_d_k, const int32_t* draft_tok,
                                                int64_t ld_x, const int32_t* parent, int32_t R, int32_t K,
                                                int32_t V, int32_t max_rows, float temperature, uint64_t seed,
                                                uint64_t round, uint64_t* round_dev, const int64_t* req_id,
                                                const int32_t* row_req, const int32_t* row_pos,
                                                const int32_t* cap, int32_t* ceiling, int32_t* accepted_len,
                                                int32_t* out_tokens, int32_t* stop_pos, float* p_x, float* q_x,
                                                int32_t* status, void* stream) {
  return verify_impl(tgt, t_dtype, ld_t, cu_seqlens, drf, d_dtype, ld_d_r, ld_d_k, draft_tok, ld_x, parent, R, K,
                     V, max_rows, temperature, seed, round, round_dev, req_id, row_req, row_pos, cap, ceiling,
                     accepted_len, out_tokens, stop_pos, p_x, q_x, status, nullptr, 0, true, stream);
}
