// Markov-head sequential stage (greedy chain) and PCTree expansion for gfx950.
//
// Operation (DSpark study notes, section 4 "Semi-Autoregressive Generation";
// PCTree article): z = L_d + U[prev] . W over the whole vocabulary, with
// U [V, r] and W [r, V] the two low-rank factors of the Markov transition
// table. The chain keeps argmax z per request; the tree keeps, per frontier
// parent, the top-k children and log-sum-exp of z, then prunes by summed
// log-probability.
//
// The contraction is the only dense GEMM on the path, so it runs on MFMA
// (v_mfma_f32_32x32x16_bf16). It is computed transposed, z^T = Wt . U[prev]^T:
// MFMA rows are vocabulary entries and MFMA columns are parent rows, so each
// lane's 16 accumulators of a 32x32 block belong to ONE parent row (column
// lane % 32) and to 16 increasing token ids. The epilogue therefore keeps
// per-lane running state (arg-max, or top-4 and an online log-sum-exp) for two
// parent rows without any cross-lane traffic per tile; lanes, waves and column
// groups are merged once at the end.
//
// Workgroup (512 threads, 8 waves as 2 vocab x 4 rows): one block of 256 parent
// rows and a strided set of 128-token vocabulary tiles (tile g, g+G, ...), so a
// Markov step over up to 256 requests streams Wt exactly once. The gathered
// U rows of its parents (256 x rank bf16) stay in LDS for all tiles; Wt is
// streamed through two 128 x 32 LDS chunks (double buffered). LDS rows are
// XOR-swizzled at 16-byte granularity so the 32 rows read by one MFMA fragment
// load hit distinct banks. Partial results per (column group, row) go to the
// workspace; small merge kernels combine them.
#include <math.h>

#include "dsp_internal.h"

namespace dsp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTV = 128;  // vocabulary entries per tile
constexpr int kWR = 4;            // wavefronts along the parent-row axis
constexpr int kTR = 64 * kWR;     // parent rows per workgroup (256)
constexpr int kGT = 128 * kWR;    // threads per workgroup: 2 (vocab) x kWR (rows) wavefronts
constexpr int kKC = 32;   // rank chunk staged per step
constexpr int kTopK = 4;  // children tracked per parent
constexpr int kTargetWGs = 256;  // one 512-thread workgroup per CU

enum { MODE_ARGMAX = 0, MODE_ARGMAX_LSE = 1, MODE_TREE = 2 };

struct ChainPart {  // per (group, row)
  uint64_t key;     // arg-max key of z (fp32), lowest id on ties
  float ref;        // log2-domain reference
  float pad;
  double sum;       // sum of exp2(z*log2e - ref)
};
struct TreePart {
  float val[kTopK];
  int32_t idx[kTopK];
  float ref;
  float pad;
  double sum;
};
static_assert(sizeof(ChainPart) == 24, "chain partial size");
static_assert(sizeof(TreePart) == 48, "tree partial size");

struct GemmArgs {
  const uint16_t* U;
  const uint16_t* Wt;
  int32_t V, rank;
  const int32_t* row_tok;  // token of parent row r at row_tok[r * ld_tok]
  int64_t ld_tok;
  const uint16_t* L;
  int64_t ldL_r, ldL_d;
  int32_t d;               // depth index of the L rows (0-based)
  int32_t rows, rows_per_req, G;
  void* part;              // ChainPart or TreePart [rows][G]
  int32_t* status;
};

// 16-byte slot of (row, vector) in a swizzled LDS tile whose rows hold `nv` vectors
// (nv a multiple of 4): the vector index is XOR-ed with the low row bits inside
// aligned groups of 8 (or 4), so consecutive rows start on different banks.
__device__ __forceinline__ int swz(int row, int kv, int nv) {
  const int m = (nv & 7) == 0 ? 7 : 3;
  return row * nv + ((kv & ~m) | ((kv ^ row) & m));
}


// (value desc, id asc) order of top-k entries
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}
__device__ __forceinline__ void cswap(float& va, int& ia, float& vb, int& ib) {
  if (better(vb, ib, va, ia)) {
    const float fv = va; va = vb; vb = fv;
    const int iv = ia; ia = ib; ib = iv;
  }
}
// Top 4 of two sorted lists of 4 (a and b, best first), written to a: the pairwise best
// of a and reversed b is a bitonic sequence holding the top 4; two half-cleaner stages
// sort it. Fixed indices only, so everything stays in registers.
__device__ __forceinline__ void merge_top4(float* va, int* ia, const float* vb, const int* ib) {
  float c[4];
  int d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool ta = better(va[q], ia[q], vb[3 - q], ib[3 - q]);
    c[q] = ta ? va[q] : vb[3 - q];
    d[q] = ta ? ia[q] : ib[3 - q];
  }
  cswap(c[0], d[0], c[2], d[2]);
  cswap(c[1], d[1], c[3], d[3]);
  cswap(c[0], d[0], c[1], d[1]);
  cswap(c[2], d[2], c[3], d[3]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    va[q] = c[q];
    ia[q] = d[q];
  }
}

template <int MODE>
__global__ __launch_bounds__(kGT, 1) void markov_gemm_kernel(GemmArgs a) {
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave & 1, wr = wave >> 1;
  const int g = blockIdx.x, rb = blockIdx.y;
  const int r0 = rb * kTR;
  const int nvu = a.rank / 8;     // 16-byte vectors per U row
  u32x4* Us = lds;                // [kTR][nvu] swizzled
  u32x4* Ws = lds + kTR * nvu;    // [2][kTV][4] swizzled
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // gather U rows of this block's parents
  for (int e = tid; e < kTR * nvu; e += kGT) {
    const int rr = e / nvu, kv = e % nvu;
    const int r = r0 + rr;
    u32x4 val = zero4;
    if (r < a.rows) {
      int tok = a.row_tok[(size_t)r * a.ld_tok];
      if (tok < 0 || tok >= a.V) {
        if (kv == 0 && g == 0) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
        tok = 0;
      }
      val = *(const u32x4*)(a.U + (size_t)tok * a.rank + kv * 8);
    }
    Us[swz(rr, kv, nvu)] = val;
  }

  // per-lane state for parent rows j = 0, 1 (row r0 + wr*64 + j*32 + lane%32)
  float best[2] = {-INFINITY, -INFINITY};
  int bidx[2] = {0x7fffffff, 0x7fffffff};
  float tv[2][kTopK];
  int ti[2][kTopK];
  float lref[2] = {-INFINITY, -INFINITY};
  double lsum[2] = {0.0, 0.0};
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < kTopK; ++q) {
      tv[j][q] = -INFINITY;
      ti[j][q] = 0x7fffffff;
    }

  const uint16_t* Lrow[2];
  bool rvalid[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = r0 + wr * 64 + j * 32 + (lane & 31);
    rvalid[j] = r < a.rows;
    const int req = rvalid[j] ? r / a.rows_per_req : 0;
    Lrow[j] = a.L + (size_t)req * a.ldL_r + (size_t)a.d * a.ldL_d;
  }

  const int ncb = (a.V + kTV - 1) / kTV;
  const int nkc = a.rank / kKC;
  const int my_tiles = g < ncb ? (ncb - g + a.G - 1) / a.G : 0;
  const int nsteps = my_tiles * nkc;  // (tile, rank chunk) pairs streamed by this workgroup
  bool l_al[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) l_al[j] = (((uintptr_t)Lrow[j]) & 7u) == 0;

  // Wt chunk of step st: 128 tokens x 32 rank values = 512 16-byte vectors over the workgroup
  constexpr int kWQ = (kTV * 4) / kGT;  // vectors per thread (1)
  auto load_w = [&](int st, u32x4* r) {
    const int t = st / nkc, kc = st - t * nkc;
    const int v0 = (g + t * a.G) * kTV;
#pragma unroll
    for (int q = 0; q < kWQ; ++q) {
      const int e = tid + q * kGT;
      const int vv = e >> 2, kv = e & 3;
      const int v = v0 + vv;
      r[q] = v < a.V ? *(const u32x4*)(a.Wt + (size_t)v * a.rank + kc * kKC + kv * 8) : zero4;
    }
  };
  auto store_w = [&](int buf, const u32x4* r) {
#pragma unroll
    for (int q = 0; q < kWQ; ++q) {
      const int e = tid + q * kGT;
      const int vv = e >> 2, kv = e & 3;
      Ws[buf * kTV * 4 + vv * 4 + (kv ^ ((vv >> 1) & 3))] = r[q];
    }
  };
  // L values of this lane for tile v0, as bf16 pairs: [row j][vocab block i][group h]
  uint2 lpre[2][2][4];
  auto load_l = [&](int v0) {
    const bool full = v0 + kTV <= a.V;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int v = v0 + wv * 64 + i * 32 + 8 * h + 4 * (lane >> 5);
          uint2 w = {0u, 0u};
          if (rvalid[j]) {
            if (full && l_al[j]) {
              w = *(const uint2*)(Lrow[j] + v);
            } else {
              uint32_t e[4];
#pragma unroll
              for (int l = 0; l < 4; ++l) e[l] = v + l < a.V ? (uint32_t)Lrow[j][v + l] : 0u;
              w.x = e[0] | (e[1] << 16);
              w.y = e[2] | (e[3] << 16);
            }
          }
          lpre[j][i][h] = w;
        }
    }
  };

  constexpr int kRing = MODE == MODE_ARGMAX ? 4 : 2;  // Wt chunks in flight per thread
  u32x4 wring[kRing][kWQ];
#pragma unroll
  for (int p = 0; p < kRing; ++p)
    if (p < nsteps) load_w(p, wring[p]);
  f32x16 acc[2][2];
  for (int base = 0; base < nsteps; base += kRing) {
#pragma unroll
    for (int p = 0; p < kRing; ++p) {
      const int st = base + p;
      if (st >= nsteps) break;  // uniform over the workgroup
      const int t = st / nkc, kc = st - t * nkc;
      const int v0 = (g + t * a.G) * kTV;
      if (kc == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        load_l(v0);
      }
      // buffer st&1 was last read two steps ago, before the previous barrier
      store_w(st & 1, wring[p]);
      __syncthreads();
      if (st + kRing < nsteps) load_w(st + kRing, wring[p]);
      const u32x4* Wb = Ws + (st & 1) * kTV * 4;
#pragma unroll
      for (int ks = 0; ks < kKC / 16; ++ks) {
        bf16x8 af[2], bu[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int vv = wv * 64 + i * 32 + (lane & 31);
          const int kv = ks * 2 + (lane >> 5);
          u32x4 tw = Wb[vv * 4 + (kv ^ ((vv >> 1) & 3))];
          af[i] = __builtin_bit_cast(bf16x8, tw);
          const int rr = wr * 64 + i * 32 + (lane & 31);
          u32x4 tu = Us[swz(rr, kc * (kKC / 8) + kv, nvu)];
          bu[i] = __builtin_bit_cast(bf16x8, tu);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bu[j], acc[i][j], 0, 0, 0);
      }
      if (kc != nkc - 1) continue;
      // epilogue: lane holds, for parent row j, tokens v0 + wv*64 + i*32 + 8*h + 4*(lane/32) + l,
      // visited in increasing token order; z = acc + L is formed on the fly (twice when the
      // log-sum-exp is needed) instead of being kept in registers
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!rvalid[j]) continue;
        float tmax = -INFINITY;
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const int i = q >> 4, h = (q >> 2) & 3, l = q & 3;
          const int v = v0 + wv * 64 + i * 32 + 8 * h + 4 * (lane >> 5) + l;
          const uint32_t w = l < 2 ? lpre[j][i][h].x : lpre[j][i][h].y;
          const float zz = v < a.V ? acc[i][j][4 * h + l] + ((l & 1) ? bf16_hi(w) : bf16_lo(w)) : -INFINITY;
          tmax = fmaxf(tmax, zz);
          if (MODE == MODE_TREE) {
            if (zz > tv[j][kTopK - 1]) {
              tv[j][kTopK - 1] = zz;
              ti[j][kTopK - 1] = v;
#pragma unroll
              for (int p = kTopK - 1; p > 0; --p) {
                if (tv[j][p] > tv[j][p - 1]) {
                  const float fv = tv[j][p]; tv[j][p] = tv[j][p - 1]; tv[j][p - 1] = fv;
                  const int iv = ti[j][p]; ti[j][p] = ti[j][p - 1]; ti[j][p - 1] = iv;
                }
              }
            }
          } else if (zz > best[j]) {
            best[j] = zz;
            bidx[j] = v;
          }
        }
        if (MODE != MODE_ARGMAX && tmax != -INFINITY) {
          const float nref = fmaxf(lref[j], tmax * kLog2e);
          float ts = 0.f;
#pragma unroll
          for (int q = 0; q < 32; ++q) {
            const int i = q >> 4, h = (q >> 2) & 3, l = q & 3;
            const int v = v0 + wv * 64 + i * 32 + 8 * h + 4 * (lane >> 5) + l;
            const uint32_t w = l < 2 ? lpre[j][i][h].x : lpre[j][i][h].y;
            const float zz = acc[i][j][4 * h + l] + ((l & 1) ? bf16_hi(w) : bf16_lo(w));
            ts += v < a.V ? fast_exp2(__builtin_fmaf(zz, kLog2e, -nref)) : 0.f;
          }
          const double scale = lref[j] == -INFINITY ? 0.0 : (double)fast_exp2(lref[j] - nref);
          lsum[j] = lsum[j] * scale + (double)ts;
          lref[j] = nref;
        }
      }
    }
  }

  // merge lane pairs (lane, lane ^ 32 hold the same parent rows)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (MODE == MODE_TREE) {
      float ov[kTopK];
      int oi[kTopK];
#pragma unroll
      for (int q = 0; q < kTopK; ++q) {
        ov[q] = __shfl_xor(tv[j][q], 32, 64);
        oi[q] = __shfl_xor(ti[j][q], 32, 64);
      }
      merge_top4(tv[j], ti[j], ov, oi);
    } else {
      const float ob = __shfl_xor(best[j], 32, 64);
      const int oi = __shfl_xor(bidx[j], 32, 64);
      if (ob > best[j] || (ob == best[j] && oi < bidx[j])) {
        best[j] = ob;
        bidx[j] = oi;
      }
    }
    if (MODE != MODE_ARGMAX) {
      const float oref = __shfl_xor(lref[j], 32, 64);
      const double osum = __shfl_xor(lsum[j], 32, 64);
      const float nref = fmaxf(lref[j], oref);
      double s = 0.0;
      if (lref[j] != -INFINITY) s += lsum[j] * exp2((double)lref[j] - (double)nref);
      if (oref != -INFINITY) s += osum * exp2((double)oref - (double)nref);
      lref[j] = nref;
      lsum[j] = s;
    }
  }

  // merge the two vocabulary waves (wv = 0, 1) through LDS, then write partials
  __syncthreads();
  if (MODE == MODE_TREE) {
    TreePart* xs = (TreePart*)lds;  // [kWR (wr)][64 rows]
    if (wv == 1 && lane < 32) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        TreePart p;
#pragma unroll
        for (int q = 0; q < kTopK; ++q) {
          p.val[q] = tv[j][q];
          p.idx[q] = ti[j][q];
        }
        p.ref = lref[j];
        p.pad = 0.f;
        p.sum = lsum[j];
        xs[wr * 64 + j * 32 + lane] = p;
      }
    }
    __syncthreads();
    if (wv == 0 && lane < 32) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = r0 + wr * 64 + j * 32 + lane;
        if (r >= a.rows) continue;
        const TreePart o = xs[wr * 64 + j * 32 + lane];
        TreePart p;
        merge_top4(tv[j], ti[j], o.val, o.idx);
#pragma unroll
        for (int q = 0; q < kTopK; ++q) {
          p.val[q] = tv[j][q];
          p.idx[q] = ti[j][q];
        }
        const float nref = fmaxf(lref[j], o.ref);
        double s = 0.0;
        if (lref[j] != -INFINITY) s += lsum[j] * exp2((double)lref[j] - (double)nref);
        if (o.ref != -INFINITY) s += o.sum * exp2((double)o.ref - (double)nref);
        p.ref = nref;
        p.pad = 0.f;
        p.sum = s;
        ((TreePart*)a.part)[(size_t)r * a.G + g] = p;
      }
    }
  } else {
    ChainPart* xs = (ChainPart*)lds;
    if (wv == 1 && lane < 32) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        ChainPart p;
        p.key = bidx[j] == 0x7fffffff ? 0ull : amax_key(best[j], (uint32_t)bidx[j]);
        p.ref = lref[j];
        p.pad = 0.f;
        p.sum = lsum[j];
        xs[wr * 64 + j * 32 + lane] = p;
      }
    }
    __syncthreads();
    if (wv == 0 && lane < 32) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = r0 + wr * 64 + j * 32 + lane;
        if (r >= a.rows) continue;
        const ChainPart o = xs[wr * 64 + j * 32 + lane];
        ChainPart p;
        const uint64_t k0 = bidx[j] == 0x7fffffff ? 0ull : amax_key(best[j], (uint32_t)bidx[j]);
        p.key = k0 > o.key ? k0 : o.key;
        const float nref = fmaxf(lref[j], o.ref);
        double s = 0.0;
        if (MODE != MODE_ARGMAX) {
          if (lref[j] != -INFINITY) s += lsum[j] * exp2((double)lref[j] - (double)nref);
          if (o.ref != -INFINITY) s += o.sum * exp2((double)o.ref - (double)nref);
        }
        p.ref = nref;
        p.pad = 0.f;
        p.sum = s;
        ((ChainPart*)a.part)[(size_t)r * a.G + g] = p;
      }
    }
  }
}

// ---------------------------------------------------------------- chain merge
struct ChainMergeArgs {
  const ChainPart* part;
  int32_t G, R, d;
  int32_t* y;
  int64_t ld_y;
  float* logq;
};

__global__ __launch_bounds__(64) void chain_merge_kernel(ChainMergeArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const ChainPart* pr = a.part + (size_t)r * a.G;
  uint64_t best = 0;
  float H = -INFINITY;
  for (int g = lane; g < a.G; g += 64) {
    best = pr[g].key > best ? pr[g].key : best;
    H = fmaxf(H, pr[g].ref);
  }
  best = wave_max(best);
  if (lane == 0) a.y[(size_t)r * a.ld_y + a.d] = (int32_t)amax_index(best);
  if (a.logq) {
    H = wave_max(H);
    double S = 0.0;
    for (int g = lane; g < a.G; g += 64)
      if (pr[g].ref != -INFINITY) S += pr[g].sum * exp2((double)pr[g].ref - (double)H);
    S = wave_sum(S);
    if (lane == 0) {
      const double lse2 = (double)H + log2(S);
      const double zy = (double)amax_value(best);
      a.logq[(size_t)r * a.ld_y + a.d] = (float)((zy * kLog2ed - lse2) * kLn2d);
    }
  }
}

// ---------------------------------------------------------------- tree merge
struct Kept {
  int32_t token;
  int32_t parent;  // kept id of the parent, -1 = root
  double score;
};

struct TreeMergeArgs {
  const TreePart* part;
  int32_t G;
  int32_t d;            // 1-based depth being expanded
  int32_t fp, fn;       // parents per request, frontier size after pruning
  int32_t topk, F, R, V, rank;
  const int32_t* ptok;  // parent tokens [R * fp] (depth 1: anchors)
  const double* pscore; // parent scores [R * fp] (NULL at depth 1)
  int32_t* ntok;        // next frontier tokens [R * fn]
  double* nscore;       // next frontier scores [R * fn]
  Kept* kept;           // [R][D * F]
  int32_t kept_stride;
  const uint16_t* L;
  int64_t ldL_r, ldL_d;
  const uint16_t* U;
  const uint16_t* Wt;
  int32_t* status;
};

// One workgroup per request: merge the column-group partials of its parents
// (one wavefront per parent), score every candidate child in fp64 (one
// wavefront per candidate, lanes splitting the rank), keep the top-F by
// (s desc, parent slot, child rank).
__global__ __launch_bounds__(256) void tree_merge_kernel(TreeMergeArgs a) {
  __shared__ double c_score[256];
  __shared__ int32_t c_tok[256];
  __shared__ double p_lse[64];
  __shared__ int32_t p_top[64][kTopK];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nc = a.fp * a.topk;
  for (int p = w; p < a.fp; p += 4) {
    const TreePart* pr = a.part + (size_t)(i * a.fp + p) * a.G;
    float tv[kTopK];
    int ti[kTopK];
#pragma unroll
    for (int q = 0; q < kTopK; ++q) {
      tv[q] = -INFINITY;
      ti[q] = 0x7fffffff;
    }
    float H = -INFINITY;
    for (int g = lane; g < a.G; g += 64) {
      merge_top4(tv, ti, pr[g].val, pr[g].idx);
      H = fmaxf(H, pr[g].ref);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov[kTopK];
      int oi[kTopK];
#pragma unroll
      for (int q = 0; q < kTopK; ++q) {
        ov[q] = __shfl_xor(tv[q], o, 64);
        oi[q] = __shfl_xor(ti[q], o, 64);
      }
      merge_top4(tv, ti, ov, oi);
    }
    H = wave_max(H);
    double S = 0.0;
    for (int g = lane; g < a.G; g += 64)
      if (pr[g].ref != -INFINITY) S += pr[g].sum * exp2((double)pr[g].ref - (double)H);
    S = wave_sum(S);
    if (lane == 0) {
      p_lse[p] = ((double)H + log2(S)) * kLn2d;
#pragma unroll
      for (int q = 0; q < kTopK; ++q) p_top[p][q] = ti[q];
    }
  }
  __syncthreads();
  for (int c = w; c < nc; c += 4) {
    const int p = c / a.topk, rk = c % a.topk;
    int v = p_top[p][rk];
    if (v < 0 || v >= a.V) {  // only reachable with non-finite scores
      if (lane == 0) atomicOr(a.status, DSP_STATUS_NONFINITE);
      v = 0;
    }
    const int ptoken = a.ptok[i * a.fp + p];
    // z_v recomputed in fp64 for the score: lanes split the rank
    const uint16_t* ur = a.U + (size_t)ptoken * a.rank;
    const uint16_t* wr = a.Wt + (size_t)v * a.rank;
    double m = 0.0;
    for (int j = lane; j < a.rank; j += 64) m += (double)bf16_val(ur[j]) * (double)bf16_val(wr[j]);
    m = wave_sum(m);
    if (lane == 0) {
      const double z = (double)bf16_val(a.L[(size_t)i * a.ldL_r + (size_t)(a.d - 1) * a.ldL_d + v]) + m;
      const double ps = a.pscore ? a.pscore[i * a.fp + p] : 0.0;
      c_score[c] = ps + fmin(0.0, z - p_lse[p]);
      c_tok[c] = v;
    }
  }
  __syncthreads();
  if (tid < nc) {
    const double s = c_score[tid];
    int rank = 0;
    for (int c = 0; c < nc; ++c) {
      const double o = c_score[c];
      rank += (o > s || (o == s && c < tid)) ? 1 : 0;  // candidate index order = (parent slot, child rank)
    }
    if (rank < a.fn) {
      const int p = tid / a.topk;
      a.ntok[i * a.fn + rank] = c_tok[tid];
      a.nscore[i * a.fn + rank] = s;
      Kept k;
      k.token = c_tok[tid];
      k.parent = a.d == 1 ? -1 : (a.d - 2) * a.F + p;
      k.score = s;
      a.kept[(size_t)i * a.kept_stride + (size_t)(a.d - 1) * a.F + rank] = k;
    }
  }
}

struct TreeFinalArgs {
  const Kept* kept;
  int32_t kept_stride, D, F, topk, topN, R;
  int32_t* node_token;
  int32_t* node_parent;
  int32_t* node_depth;
  double* node_score;
  int32_t* n_nodes;
};

__global__ __launch_bounds__(256) void tree_final_kernel(TreeFinalArgs a) {
  __shared__ double s_score[1024];
  __shared__ int32_t s_valid[1024];
  __shared__ int32_t s_out[1024];
  __shared__ int32_t fsz[1024];
  const int i = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) {
    int prev = 1;  // frontier size after depth d: min(F, topk * previous)
    for (int d = 0; d < a.D; ++d) {
      const int c = a.topk * prev;
      fsz[d] = c < a.F ? c : a.F;
      prev = fsz[d];
    }
  }
  __syncthreads();
  const int nk = a.D * a.F;
  const Kept* kr = a.kept + (size_t)i * a.kept_stride;
  for (int e = tid; e < nk; e += 256) {
    const int d = e / a.F, slot = e % a.F;
    s_valid[e] = slot < fsz[d] ? 1 : 0;
    s_score[e] = s_valid[e] ? kr[e].score : 0.0;
    s_out[e] = -1;
  }
  __syncthreads();
  // rank by (score desc, depth asc, slot asc) == (score desc, kept id asc)
  for (int e = tid; e < nk; e += 256) {
    if (!s_valid[e]) continue;
    const double s = s_score[e];
    int rank = 0;
    for (int o = 0; o < nk; ++o)
      rank += (s_valid[o] && (s_score[o] > s || (s_score[o] == s && o < e))) ? 1 : 0;
    if (rank < a.topN) s_out[e] = rank;
  }
  __syncthreads();
  int total = 0;
  for (int d = 0; d < a.D; ++d) total += fsz[d];
  const int nout = total < a.topN ? total : a.topN;
  for (int e = tid; e < nk; e += 256) {
    const int o = s_out[e];
    if (o < 0) continue;
    const Kept k = kr[e];
    const size_t at = (size_t)i * a.topN + o;
    a.node_token[at] = k.token;
    a.node_parent[at] = k.parent < 0 ? -1 : s_out[k.parent];
    a.node_depth[at] = e / a.F + 1;
    a.node_score[at] = k.score;
  }
  for (int o = nout + tid; o < a.topN; o += 256) {
    const size_t at = (size_t)i * a.topN + o;
    a.node_token[at] = -1;
    a.node_parent[at] = -1;
    a.node_depth[at] = 0;
    a.node_score[at] = 0.0;
  }
  if (tid == 0) a.n_nodes[i] = nout;
}

size_t gemm_lds_bytes(int rank) { return (size_t)(kTR * (rank / 8) + 2 * kTV * 4) * 16; }
static_assert((kTV * 4) % kGT == 0, "Wt chunk must split evenly over the workgroup");

int pick_groups(int rows, int V) {
  const int nrb = (rows + kTR - 1) / kTR;
  const int ncb = (V + kTV - 1) / kTV;
  int G = (kTargetWGs + nrb - 1) / nrb;
  if (G > ncb) G = ncb;
  if (G < 1) G = 1;
  return G;
}

template <int MODE>
int32_t launch_gemm(int kid, const GemmArgs& a, hipStream_t s) {
  const size_t lds = gemm_lds_bytes(a.rank);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)markov_gemm_kernel<MODE>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  dim3 grid(a.G, (a.rows + kTR - 1) / kTR);
  launch(kid, markov_gemm_kernel<MODE>, grid, dim3(kGT), (uint32_t)lds, s, a);
  return hip_check(hipGetLastError(), "markov gemm launch");
}

int32_t check_markov_common(const void* L, int32_t l_dtype, const void* U, const void* Wt, int32_t V,
                            int32_t rank) {
  if (l_dtype != DSP_BF16) return fail(DSP_ERR_DTYPE, "L must be bf16");
  if (!L || !U || !Wt) return fail(DSP_ERR_NULL, "L, U and Wt are required");
  if (V < 1) return fail(DSP_ERR_SHAPE, "V must be >= 1");
  if (rank < 32 || rank > 512 || rank % 32) return fail(DSP_ERR_SHAPE, "rank must be a multiple of 32 in [32, 512]");
  if (((uintptr_t)U) % 16 || ((uintptr_t)Wt) % 16) return fail(DSP_ERR_ALIGN, "U and Wt must be 16-byte aligned");
  if (((uintptr_t)L) % 2) return fail(DSP_ERR_ALIGN, "L must be 2-byte aligned");
  return DSP_OK;
}

// Frontier size after each depth: f_d = min(F, k * f_{d-1}), f_0 = 1.
void frontier_sizes(int D, int topk, int F, int* f) {
  int prev = 1;
  for (int d = 0; d < D; ++d) {
    const long c = (long)topk * prev;
    f[d] = (int)(c < F ? c : F);
    prev = f[d];
  }
}

struct TreeLayout {
  size_t off_part, off_tok0, off_tok1, off_sc0, off_sc1, off_kept, total;
  int kept_stride;
};
TreeLayout tree_layout(int R, int D, int V, int rank, int topk, int F) {
  (void)rank;
  TreeLayout t;
  int f[1024];
  frontier_sizes(D, topk, F, f);
  size_t part = 0;
  int fp = 1;
  for (int d = 0; d < D; ++d) {
    const int rows = R * fp;
    const size_t b = (size_t)pick_groups(rows, V) * rows * sizeof(TreePart);
    part = b > part ? b : part;
    fp = f[d];
  }
  size_t off = 0;
  t.off_part = off; off = align_up(off + part, 256);
  t.off_tok0 = off; off = align_up(off + (size_t)R * F * 4, 256);
  t.off_tok1 = off; off = align_up(off + (size_t)R * F * 4, 256);
  t.off_sc0 = off; off = align_up(off + (size_t)R * F * 8, 256);
  t.off_sc1 = off; off = align_up(off + (size_t)R * F * 8, 256);
  t.kept_stride = D * F;
  t.off_kept = off; off = align_up(off + (size_t)R * D * F * sizeof(Kept), 256);
  t.total = off;
  return t;
}

}  // namespace
}  // namespace dsp

using namespace dsp;

extern "C" size_t dsp_draft_markov_step_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps,
                                                       int32_t want_logq) {
  (void)rank;
  (void)n_steps;
  (void)want_logq;
  if (R < 1 || V < 1) return 0;
  return align_up((size_t)pick_groups(R, V) * R * sizeof(ChainPart), 256);
}

extern "C" int32_t dsp_draft_markov_step(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                                         const void* U, const void* Wt, int32_t V, int32_t rank,
                                         const int32_t* prev_tok, int32_t R, int32_t n_steps, int32_t* y,
                                         int64_t ld_y, float* logq, int32_t* status, void* ws,
                                         size_t ws_bytes, void* stream) {
  clear_error();
  int32_t rc = check_markov_common(L, l_dtype, U, Wt, V, rank);
  if (rc) return rc;
  if (R < 1 || n_steps < 1) return fail(DSP_ERR_SHAPE, "need R >= 1 and n_steps >= 1");
  if (!prev_tok || !y || !status) return fail(DSP_ERR_NULL, "prev_tok, y and status are required");
  if (ld_y < n_steps) return fail(DSP_ERR_SHAPE, "ld_y < n_steps");
  if (ldL_d < V || ldL_r < (int64_t)(n_steps - 1) * ldL_d + V) return fail(DSP_ERR_SHAPE, "L strides too small");
  const size_t need = dsp_draft_markov_step_workspace_size(R, V, rank, n_steps, logq != nullptr);
  if (!ws || ws_bytes < need) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  hipStream_t s = (hipStream_t)stream;
  const int G = pick_groups(R, V);
  for (int d = 0; d < n_steps; ++d) {
    GemmArgs ga{(const uint16_t*)U, (const uint16_t*)Wt, V, rank,
                d == 0 ? prev_tok : y + (d - 1), d == 0 ? 1 : ld_y,
                (const uint16_t*)L, ldL_r, ldL_d, d, R, 1, G, ws, status};
    rc = logq ? launch_gemm<MODE_ARGMAX_LSE>(DSP_K_MARKOV_GEMM, ga, s)
              : launch_gemm<MODE_ARGMAX>(DSP_K_MARKOV_GEMM, ga, s);
    if (rc) return rc;
    ChainMergeArgs ma{(const ChainPart*)ws, G, R, d, y, ld_y, logq};
    launch(DSP_K_MARKOV_MERGE, chain_merge_kernel, dim3(R), dim3(64), 0, s, ma);
    rc = hip_check(hipGetLastError(), "chain merge launch");
    if (rc) return rc;
  }
  return DSP_OK;
}

extern "C" size_t dsp_tree_expand_workspace_size(int32_t R, int32_t D, int32_t V, int32_t rank, int32_t topk,
                                                 int32_t frontier, int32_t topN) {
  (void)topN;
  if (R < 1 || D < 1 || V < 1 || topk < 1 || frontier < 1 || D * frontier > 1024) return 0;
  return tree_layout(R, D, V, rank, topk, frontier).total;
}

extern "C" int32_t dsp_tree_expand(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                                   const void* U, const void* Wt, int32_t V, int32_t rank,
                                   const int32_t* anchor, int32_t R, int32_t D, int32_t topk,
                                   int32_t frontier, int32_t topN, int32_t* node_token,
                                   int32_t* node_parent, int32_t* node_depth, double* node_score,
                                   int32_t* n_nodes, int32_t* status, void* ws, size_t ws_bytes,
                                   void* stream) {
  clear_error();
  int32_t rc = check_markov_common(L, l_dtype, U, Wt, V, rank);
  if (rc) return rc;
  if (R < 1 || D < 1) return fail(DSP_ERR_SHAPE, "need R >= 1 and D >= 1");
  if (topk < 1 || topk > kTopK || topk > V) return fail(DSP_ERR_SHAPE, "need 1 <= topk <= min(4, V)");
  if (frontier < 1 || frontier > 64 || topk * frontier > 256 || D * frontier > 1024)
    return fail(DSP_ERR_SHAPE, "need 1 <= frontier <= 64, topk*frontier <= 256, D*frontier <= 1024");
  if (topN < 1 || topN > 1024) return fail(DSP_ERR_SHAPE, "need 1 <= topN <= 1024");
  if (!anchor || !node_token || !node_parent || !node_depth || !node_score || !n_nodes || !status)
    return fail(DSP_ERR_NULL, "required pointer is NULL");
  if (ldL_d < V || ldL_r < (int64_t)(D - 1) * ldL_d + V) return fail(DSP_ERR_SHAPE, "L strides too small");
  const TreeLayout T = tree_layout(R, D, V, rank, topk, frontier);
  if (!ws || ws_bytes < T.total) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", T.total);
  hipStream_t s = (hipStream_t)stream;
  const uintptr_t b = (uintptr_t)ws;
  TreePart* part = (TreePart*)(b + T.off_part);
  int32_t* tok[2] = {(int32_t*)(b + T.off_tok0), (int32_t*)(b + T.off_tok1)};
  double* sc[2] = {(double*)(b + T.off_sc0), (double*)(b + T.off_sc1)};
  Kept* kept = (Kept*)(b + T.off_kept);
  int f[1024];
  frontier_sizes(D, topk, frontier, f);
  int fp = 1;
  for (int d = 1; d <= D; ++d) {
    const int rows = R * fp;
    const int G = pick_groups(rows, V);
    const int32_t* ptok = d == 1 ? anchor : tok[d & 1];
    GemmArgs ga{(const uint16_t*)U, (const uint16_t*)Wt, V, rank, ptok, 1, (const uint16_t*)L, ldL_r,
                ldL_d, d - 1, rows, fp, G, part, status};
    rc = launch_gemm<MODE_TREE>(DSP_K_TREE_GEMM, ga, s);
    if (rc) return rc;
    const int fn = f[d - 1];
    TreeMergeArgs ma{part, G, d, fp, fn, topk, frontier, R, V, rank, ptok, d == 1 ? nullptr : sc[d & 1],
                     tok[(d + 1) & 1], sc[(d + 1) & 1], kept, T.kept_stride, (const uint16_t*)L, ldL_r,
                     ldL_d, (const uint16_t*)U, (const uint16_t*)Wt, status};
    launch(DSP_K_TREE_MERGE, tree_merge_kernel, dim3(R), dim3(256), 0, s, ma);
    rc = hip_check(hipGetLastError(), "tree merge launch");
    if (rc) return rc;
    fp = fn;
  }
  TreeFinalArgs fa{kept, T.kept_stride, D, frontier, topk, topN, R, node_token, node_parent, node_depth,
                   node_score, n_nodes};
    launch(DSP_K_TREE_FINAL, tree_final_kernel, dim3(R), dim3(256), 0, s, fa);
  return hip_check(hipGetLastError(), "tree final launch");
}
