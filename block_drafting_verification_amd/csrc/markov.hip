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
// Workgroup (512 threads, 8 waves): 256 parent rows, one 32-row MFMA column
// block per wave, and a contiguous range of 32-token vocabulary stages. Each
// lane keeps its parent row's U fragments (the MFMA B operand) in registers for
// the whole launch. Wt rows and the matching L entries of a stage arrive with
// bounds-checked 16-byte buffer loads into a ring of register buffers three stages deep, are
// written to one of two LDS stage buffers and read back as MFMA A fragments
// (Wt, XOR-swizzled at 16-byte granularity so the 8 rows of a fragment read hit
// distinct bank groups) and as the epilogue's L values. One barrier per stage.
// With more than 256 parent rows (the tree), the row blocks that share a
// vocabulary range are placed on one XCD so the range's Wt is fetched into that
// XCD's L2 once. Partial results per (vocabulary range, row) go to the
// workspace; small merge kernels combine them.
#include <math.h>

#include <type_traits>

#include "dsp_internal.h"

namespace dsp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kGT = 64 * kWaves;  // threads per workgroup
constexpr int kTR = 32 * kWaves;  // parent rows per workgroup: one 32-row MFMA column block per wave
constexpr int kTS = 32;           // vocabulary entries per pipeline stage (one 32-row MFMA block)
constexpr int kTopK = 4;          // children tracked per parent
constexpr int kTargetWGs = 256;   // one workgroup per CU
static_assert(kTargetWGs <= 256, "the merge kernels read at most four partials per lane (G <= 256)");
constexpr int kZS = 144;          // bytes per row of a wave's staging tile of emitted logits (128 + pad)

enum { MODE_ARGMAX = 0, MODE_ARGMAX_LSE = 1, MODE_TREE = 2, MODE_SAMPLE = 3 };

// ---------------------------------------------------------------- streaming loads
// The stage ring is fed by raw buffer loads issued from inline assembly with explicit
// s_waitcnt vmcnt(N): the compiler's own wait insertion cannot follow loads carried
// around a loop in a register ring and drains every load in flight at the loop edge,
// which turns a 4-deep pipeline into a stop-and-go one. A buffer descriptor holds a
// base and a byte extent; the hardware returns zero for any offset at or past the
// extent, so out-of-range lanes take an offset past every extent and need no branch.
typedef uint32_t s32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;  // past every extent (extents are < 2^31 bytes)

__device__ __forceinline__ s32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  s32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  d.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);  // stride 0
  d.z = __builtin_amdgcn_readfirstlane(bytes);
  d.w = 0x00020000u;  // 32-bit data format, as for every gfx9 buffer access
  return d;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t as_rsrc(const s32x4& d) {
  void* base = (void*)(((uint64_t)d.y << 32) | d.x);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)d.z, (int)d.w);
}
// ASYNC: the inline-assembly form, whose result must not be read before a vm_wait that
// covers it. Otherwise the compiler's own buffer load (it waits where needed). Kernels
// that spill registers must use the latter: a spill could copy a register whose load
// has not landed.
// The destination is a read-write operand: the register then stays bound to its ring
// slot for the whole loop, so the compiler never hands it to another value while a
// load into it is still in flight.
// Each load starts with s_nop 4: a vector memory instruction that reads an SGPR written
// by a VALU instruction (v_readlane / v_readfirstlane, e.g. when the compiler reloads a
// spilled descriptor) needs 5 wait states in between, which the compiler inserts before
// its own memory instructions but not before inline assembly. Without them the load can
// take a stale descriptor.
template <bool ASYNC, int IMM = 0>
__device__ __forceinline__ void buf_load_x4(u32x4& v, const s32x4& d, uint32_t off) {
  static_assert(IMM >= 0 && IMM < 4096, "buffer instruction offset");
  if (ASYNC)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3"
                 : "+v"(v) : "v"(off), "s"(d), "n"(IMM) : "memory");
  else
    v = __builtin_amdgcn_raw_buffer_load_b128(as_rsrc(d), off + IMM, 0, 0);
}
template <bool ASYNC>
__device__ __forceinline__ void buf_load_u16(uint32_t& v, const s32x4& d, uint32_t off) {
  if (ASYNC)
    asm volatile("s_nop 4\n\tbuffer_load_ushort %0, %1, %2, 0 offen" : "+v"(v) : "v"(off), "s"(d) : "memory");
  else
    v = __builtin_amdgcn_raw_buffer_load_b16(as_rsrc(d), off, 0, 0);
}
template <bool ASYNC, int IMM = 0>
__device__ __forceinline__ void buf_load_x1(uint32_t& v, const s32x4& d, uint32_t off) {
  static_assert(IMM >= 0 && IMM < 4096, "buffer instruction offset");
  if (ASYNC)
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2, 0 offen offset:%3"
                 : "+v"(v) : "v"(off), "s"(d), "n"(IMM) : "memory");
  else
    v = __builtin_amdgcn_raw_buffer_load_b32(as_rsrc(d), off + IMM, 0, 0);
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// A register written by an asynchronous load is only tied to the load statement: plain
// arithmetic that reads it (bit tests, shifts, packing) could legally be scheduled above
// the vm_wait that covers the load, since the wait names no register. Passing the
// register through an empty volatile statement right after the wait makes every later
// reader depend on that statement, and volatile statements keep their program order, so
// no reader can move above the wait. It emits no instruction.
__device__ __forceinline__ void landed(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void landed(uint32_t& v) { asm volatile("" : "+v"(v)); }

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
  int32_t nrb;             // row blocks of kTR rows
  int32_t xcd_map;         // 1: row blocks of a slice share an XCD (G % 8 == 0)
  // sampled chain: the step's logits rounded to bf16 go to zout (element (row, v) at
  // zout + row*ldz_r + d*ldz_d + v), and the log-sum-exp partials are of those rounded
  // values times cz = log2(e) / T
  uint16_t* zout;
  int64_t ldz_r, ldz_d;
  float cz;
  // tree: per parent row, a value t with every entry of the row's top 4 strictly above
  // it (or NULL: no bound); entries at or below t are not offered to the top-4 list
  const float* theta;
  // rows of U the parent rows may name (0: V, the token table). The RNN head passes its
  // memo rows here (row r of the memo table for parent row r).
  int32_t u_rows;
  // base logits stored token-major (chain, one row per request): element (request i,
  // token v) of depth d at L + i + d*ldL_d + v*ldL_r, i.e. ldL_r is then the stride
  // between tokens; a stage's tile of 32 tokens x 256 requests is one contiguous read
  int32_t l_tm;
};

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

// Tree epilogue of one stage for this lane's parent row: z holds 16 tokens of the row
// (value q is token v0 + 8*(q>>2) + 4*(lane>>5) + (q&3)), tm is their maximum and ts the
// sum of exp2(z log2e - lref) against the reference of the stages before. The reference
// is raised only when the stage could exceed it by more than 2^64 (each term stays finite
// in fp32), which recomputes the stage's sum (always on a lane's first non-empty stage).
// Then the top-4 insertion, skipped unless the stage has an entry above the threshold
// thr = max(4th kept value, row bound th_row). Split in two: the branch-free part that
// adds the stage's sum (returns whether it did), and the rest.
__device__ __forceinline__ bool tree_stage_sum(float tm, float ts, float lref, double& lsum) {
  // the sum is selected, not branched on, so that the exponentials stay between the
  // MFMAs (a branch lets the compiler sink them past the whole stage)
  const bool fast = lref != -INFINITY && tm * kLog2e <= lref + 64.f;
  lsum += fast ? (double)ts : 0.0;
  return fast;
}
__device__ __forceinline__ void tree_stage_rest(bool fast, int v0, int lane, const f32x16& z, float tm, float& lref,
                                                double& lsum, float (&tv)[kTopK], int (&ti)[kTopK], float& thr,
                                                float th_row) {
  if (!fast && tm != -INFINITY) {
    const float nref = fmaxf(lref, tm * kLog2e);
    float t2 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) t2 += fast_exp2(__builtin_fmaf(z[q], kLog2e, -nref));
    const double scale = lref == -INFINITY ? 0.0 : (double)fast_exp2(lref - nref);
    lsum = lsum * scale + (double)t2;
    lref = nref;
  }
  if (tm > thr) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (z[q] > thr) {
        tv[kTopK - 1] = z[q];
        ti[kTopK - 1] = v0 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
#pragma unroll
        for (int p2 = kTopK - 1; p2 > 0; --p2) {
          if (tv[p2] > tv[p2 - 1]) {
            const float fv = tv[p2]; tv[p2] = tv[p2 - 1]; tv[p2 - 1] = fv;
            const int iv = ti[p2]; ti[p2] = ti[p2 - 1]; ti[p2 - 1] = iv;
          }
        }
        thr = fmaxf(tv[kTopK - 1], th_row);
      }
    }
  }
}
__device__ __forceinline__ void tree_stage_end(int v0, int lane, const f32x16& z, float tm, float ts, float& lref,
                                               double& lsum, float (&tv)[kTopK], int (&ti)[kTopK], float& thr,
                                               float th_row) {
  const bool fast = tree_stage_sum(tm, ts, lref, lsum);
  tree_stage_rest(fast, v0, lane, z, tm, lref, lsum, tv, ti, thr, th_row);
}

// Lanes l and l ^ 32 hold the same parent row: merge their top-4 lists, and their
// log-sum-exp pairs (reference, sum) on a common reference.
__device__ __forceinline__ void merge_pair_top4(float (&tv)[kTopK], int (&ti)[kTopK]) {
  float ov[kTopK];
  int oi[kTopK];
#pragma unroll
  for (int q = 0; q < kTopK; ++q) {
    ov[q] = __shfl_xor(tv[q], 32, 64);
    oi[q] = __shfl_xor(ti[q], 32, 64);
  }
  merge_top4(tv, ti, ov, oi);
}
__device__ __forceinline__ void merge_pair_lse(float& lref, double& lsum) {
  const float oref = __shfl_xor(lref, 32, 64);
  const double osum = __shfl_xor(lsum, 32, 64);
  const float nref = fmaxf(lref, oref);
  double s = 0.0;
  if (lref != -INFINITY) s += lsum * exp2((double)lref - (double)nref);
  if (oref != -INFINITY) s += osum * exp2((double)oref - (double)nref);
  lref = nref;
  lsum = s;
}

template <int MODE, int KS, bool LAL, bool LTM = false>
__global__ __launch_bounds__(kGT, 1) void markov_gemm_kernel(GemmArgs a) {
  constexpr int NV = 2 * KS;                  // 16-byte vectors per staged Wt row (rank padded to 16*KS)
  constexpr int WST = kTS * NV;               // Wt vectors per stage
  constexpr int WQ = (WST + kGT - 1) / kGT;   // Wt vectors loaded per thread per stage
  constexpr int LST = kTR * 4;                // L vectors per stage: 256 rows x 32 tokens
  constexpr int LQ = LST / kGT;               // L vectors loaded per thread per stage
  constexpr int NR = KS <= 16 && LAL ? 3 : 2;  // stages in flight per thread (register ring)
  constexpr int NU = NR % 2 ? 2 * NR : NR;     // stages per unrolled loop body (ring slot and
                                               // buffer parity both static)
  // asynchronous ring loads (kernels that do not spill). The sampled chain's global
  // stores share the vector memory counter with the ring's loads and may retire in any
  // order relative to them, but loads return in order among themselves: with at most
  // (NR-1)*LPS operations outstanding, the loads of the oldest stage cannot still be
  // pending (every later stage's loads would be too, more than that count), so the
  // counted waits stay sufficient; stores still in flight only make them wait longer.
  constexpr bool AS = KS <= 16;
  static_assert(LST % kGT == 0, "L stage must split evenly over the workgroup");
  extern __shared__ u32x4 lds[];              // [2][WST + LST]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // workgroup -> (vocabulary slice g, row block rb). With several row blocks, the
  // blocks sharing a slice get ids congruent mod 8 (one XCD) and adjacent in dispatch
  // order, so the slice's Wt lines are fetched once into that XCD's L2.
  int g, rb;
  {
    const int id = blockIdx.x;
    if (a.xcd_map) {
      const int j = id >> 3;
      g = (j / a.nrb) * 8 + (id & 7);
      rb = j % a.nrb;
    } else {
      g = id % a.G;
      rb = id / a.G;
    }
  }
  const int r0 = rb * kTR;
  const int nst_all = (a.V + kTS - 1) / kTS;
  const int s_begin = (int)(((long)g * nst_all) / a.G);
  const int nst = (int)(((long)(g + 1) * nst_all) / a.G) - s_begin;

  // B operand: this lane's parent row (one per lane pair) and its U row, held in
  // registers for the whole launch: k-step ks covers rank 16ks + 8*(lane/32) .. +8
  const int nloc = wave * 32 + (lane & 31);
  const int row = r0 + nloc;
  const bool rvalid = row < a.rows;
  const bool all_rows = r0 + kTR <= a.rows;  // every row of the block is a parent row
  // the row's token; its U row is fetched after the first stage's loads are issued
  int tok = 0;
  if (rvalid) {
    tok = a.row_tok[(size_t)row * a.ld_tok];
    if (tok < 0 || tok >= (a.u_rows > 0 ? a.u_rows : a.V)) {
      if (g == 0 && lane < 32) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
      tok = 0;
    }
  }
  u32x4 ufr[KS] = {};  // B fragments, loaded straight into their registers
  // the L k-step's B fragment: 1.0 (bf16) at k = this row's request within the block
  u32x4 onehot = {0u, 0u, 0u, 0u};
  if (MODE == MODE_TREE && rvalid) {
    const int j = row / a.rows_per_req - r0 / a.rows_per_req - 8 * (lane >> 5);
    if (j >= 0 && j < 8) onehot[j >> 1] = 0x3f80u << (16 * (j & 1));
  }
  // issued like the ring's loads (the compiler would otherwise keep them "pending" around
  // the stage loop and drain the ring for them); the first stage's wait covers them
  auto load_u = [&]() {
    const s32x4 udesc = make_desc(a.U, (uint32_t)((size_t)(a.u_rows > 0 ? a.u_rows : a.V) * a.rank * 2));
    const uint32_t ubase = (uint32_t)(((size_t)tok * a.rank + 8 * (lane >> 5)) * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool ok = rvalid && 16 * ks + 8 * (lane >> 5) < a.rank;
      buf_load_x4<AS>(ufr[ks], udesc, ok ? ubase + 32 * ks : kOOB);
    }
  };

  // L rows staged by this thread: row (tid + q*kGT) / 4, 16-byte column tid % 4, addressed
  // from the first request of this row block (spans checked on the host)
  const s32x4 wdesc = make_desc(a.Wt, (uint32_t)((size_t)a.V * a.rank * 2));
  const int req0 = r0 / a.rows_per_req;
  const int rlast = (r0 + kTR < a.rows ? r0 + kTR : a.rows) - 1;
  // token-major: the block's requests r0..rlast of every token (a multiple of 8 of them,
  // checked on the host), so 16-byte vectors of 8 requests are either all inside or past it
  // Row-major: up to the block's last row's token V-1. The range check of a buffer load
  // is per dword, so with V odd the dword holding that last entry would read as zero:
  // 16-byte loads (LAL: a 16-byte aligned base) extend the extent to the end of that
  // dword (2 more bytes, in the same dword, so in memory the row's own entries reach);
  // 2-byte loads keep it exact.
  const s32x4 ldesc =
      LTM ? make_desc(a.L + (size_t)r0 + (size_t)a.d * a.ldL_d,
                      (uint32_t)(((size_t)(a.V - 1) * a.ldL_r + (rlast - r0 + 1)) * 2))
          : make_desc(a.L + (size_t)req0 * a.ldL_r + (size_t)a.d * a.ldL_d,
                      (uint32_t)((((size_t)(rlast / a.rows_per_req - req0) * a.ldL_r + a.V) * 2 + (LAL ? 3 : 0)) &
                                 ~(size_t)(LAL ? 3 : 0)));
  // Tree blocks spanning at most 16 requests add the base logits through the matrix
  // cores: one extra k-step (A = the stage's 32 tokens x 16 requests of L, B = each
  // row's one-hot request), issued first so z keeps its summation order, in place of
  // unpacking a per-row L tile into the accumulators. The stage's L tile then holds one
  // row per request, transposed (token-major, 32 bytes per token).
  const bool lk = MODE == MODE_TREE && LAL && rlast / a.rows_per_req - req0 < 16;
  // Byte offsets of this thread's loads, less a per-stage term that is uniform over the
  // workgroup. Entries that are never valid (rank padding, spare threads, rows past the
  // block) start at kOOB; a stage past the range gets the term kOOB. Either way the sum
  // lies past the extent (extents and live terms are below 2^31) and the load reads zero,
  // as does a live stage's entry whose token is past V (offset past the Wt extent), while
  // an L entry past V of a row reads the next row's start or zero: masked at use.
  uint32_t wofs[WQ], lofs[LQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int e = tid + q * kGT;
    const int vv = e / NV, kv = e % NV;
    wofs[q] = e < WST && kv * 8 < a.rank ? (uint32_t)((vv * a.rank + kv * 8) * 2) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < LQ; ++q) {
    const int rr = r0 + ((tid + q * kGT) >> 2);
    lofs[q] = rr < a.rows ? (uint32_t)(((size_t)(rr / a.rows_per_req - req0) * a.ldL_r + 8 * (tid & 3)) * 2)
                          : kOOB;
    if (LTM) {  // vector e: token e / 32 of the stage, requests 8 (e % 32) .. + 8
      const int e = tid + q * kGT, rg = e & 31;
      lofs[q] = r0 + 8 * rg < a.rows ? (uint32_t)(((size_t)(e >> 5) * a.ldL_r + 8 * rg) * 2) : kOOB;
    }
    if (lk)  // request tid/4 of the block, 16-byte column tid%4; past the block's requests: zero
      lofs[q] = q == 0 && tid < 64 && (tid >> 2) <= rlast / a.rows_per_req - req0
                    ? (uint32_t)(((size_t)(tid >> 2) * a.ldL_r + 8 * (tid & 3)) * 2)
                    : kOOB;
  }
  // Every thread issues the same LPS loads for every stage, including the stages past
  // its range: the count of loads in flight is then a constant the ring's waits can name.
  constexpr int LPS = WQ + LQ * (LAL ? 1 : 8);  // loads per stage per thread
  auto load_stage = [&](int s, u32x4* rw, u32x4* rl, uint32_t (*ru)[8]) {
    const bool live = s < nst;
    const uint32_t tw = live ? (uint32_t)((size_t)(s_begin + s) * kTS * a.rank * 2) : kOOB;
    const uint32_t tl = live ? (uint32_t)((LTM ? (size_t)(s_begin + s) * kTS * a.ldL_r : (size_t)(s_begin + s) * kTS) * 2)
                             : kOOB;
#pragma unroll
    for (int q = 0; q < WQ; ++q) buf_load_x4<AS>(rw[q], wdesc, wofs[q] + tw);
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      if (LAL) {
        buf_load_x4<AS>(rl[q], ldesc, lofs[q] + tl);
      } else {
        // unaligned rows: one 2-byte load per entry, packed only after the stage's wait
#pragma unroll
        for (int l = 0; l < 8; ++l) buf_load_u16<AS>(ru[q][l], ldesc, lofs[q] + tl + 2 * l);
      }
    }
  };
  // LDS layouts. Wt stage: token row m holds NV vectors, vector kv at m*NV + swz_w(m, kv).
  // A 16-byte read by 64 lanes is served 16 lanes (256 bytes, all 64 banks) at a time,
  // so the 16 rows read together must fall on 16 distinct 16-byte slots of a 256-byte
  // window: XOR the vector index with the row within aligned groups of W = min(NV, 16)
  // vectors, R = 16 / W rows sharing a window. L stage: row n holds 4 vectors, vector c
  // at n*4 + (c ^ ((n >> 2) & 3)), so the epilogue's 8-byte reads of 16 consecutive rows
  // hit 16 distinct slots.
  auto swz_w = [](int m, int kv) {
    constexpr int W = NV < 16 ? NV : 16, R = 16 / W;
    return (kv & ~(W - 1)) | ((kv ^ (m / R)) & (W - 1));
  };
  auto store_stage = [&](int b, const u32x4* rw, const u32x4* rl, const uint32_t (*ru)[8]) {
    u32x4* Ws = lds + b * (WST + LST);
    u32x4* Ls = Ws + WST;
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int e = tid + q * kGT;
      if (e < WST) {
        const int vv = e / NV, kv = e % NV;
        Ws[vv * NV + swz_w(vv, kv)] = rw[q];
      }
    }
    if (lk) {
      // transposed: token t of request j at Lt[t * 16 + j]; every one of the 16 request
      // columns is written (zeros past the block's requests), so no stale LDS contents
      // meet the one-hot zeros. A non-finite entry is staged as -max (a zero weight times
      // an infinity would make NaN in every other request's sum): for a masked -inf that
      // ranks and weighs the same; +inf and NaN are faults and set the status bit.
      if (tid < 64) {
        uint16_t* Lt = (uint16_t*)Ls;
        const int j = tid >> 2, c = tid & 3;
        const u32x4 w = rl[0];
        bool fault = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint16_t h = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          if ((h & 0x7f80u) == 0x7f80u) {
            fault |= !(h & 0x8000u) || (h & 0x7fu);
            h = 0xff7fu;
          }
          Lt[(8 * c + e) * 16 + j] = h;
        }
        if (fault) atomicOr(a.status, DSP_STATUS_NONFINITE);
      }
      return;
    }
    if (LTM) {  // token-major tile [32 tokens][256 requests], stored as loaded
#pragma unroll
      for (int q = 0; q < LQ; ++q) Ls[tid + q * kGT] = rl[q];
      return;
    }
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      const int n = (tid + q * kGT) >> 2, c = tid & 3;
      u32x4 w;
      if (LAL) {
        w = rl[q];
      } else {
        w.x = ru[q][0] | (ru[q][1] << 16);
        w.y = ru[q][2] | (ru[q][3] << 16);
        w.z = ru[q][4] | (ru[q][5] << 16);
        w.w = ru[q][6] | (ru[q][7] << 16);
      }
      Ls[n * 4 + (c ^ ((n >> 2) & 3))] = w;
    }
  };

  // per-lane running state of this lane's parent row
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  int bcode = -1;  // chain: 16 * stage + value index of best
  float tv[kTopK];
  int ti[kTopK];
#pragma unroll
  for (int q = 0; q < kTopK; ++q) {
    tv[q] = -INFINITY;
    ti[q] = 0x7fffffff;
  }
  float lref = -INFINITY;
  double lsum = 0.0;
  // tree: an entry enters the top-4 list only above thr = max(4th kept value, row bound)
  float th_row = -INFINITY;
  if (MODE == MODE_TREE && a.theta && rvalid) th_row = a.theta[row];
  float thr = th_row;

  u32x4 ringw[NR][WQ] = {}, ringl[NR][LQ] = {};
  uint32_t ringu[NR][LAL ? 1 : LQ][8] = {};
  // prologue: stage 0, then the U rows (which wait on the token load), then the rest of
  // the ring; the first stage's wait then covers stage 0 and the U rows only
  load_stage(0, ringw[0], ringl[0], ringu[0]);
  load_u();
#pragma unroll
  for (int p = 1; p < NR; ++p) load_stage(p, ringw[p], ringl[p], ringu[p]);

  // Accumulator a of this lane is token v0 + 8*(a/4) + 4*(lane/32) + a%4 of its row, so
  // the 16 values are visited in increasing token order. The accumulator starts from
  // L (or -inf for a token past V or a row past the block), so the MFMAs leave z itself.
  auto init_from_l = [&](int s, const u32x4* Ls, f32x16& acc) {
    const int v0 = (s_begin + s) * kTS;
    uint2 w[4];
    if (LTM) {  // this lane's 16 tokens of its request, 2 bytes each from the [token][request] tile
      const uint16_t* Lt = (const uint16_t*)Ls + nloc;
      uint32_t hv[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) hv[q] = Lt[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * kTR];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        w[h].x = hv[4 * h] | (hv[4 * h + 1] << 16);
        w[h].y = hv[4 * h + 2] | (hv[4 * h + 3] << 16);
      }
    } else {
      const char* lb = (const char*)(Ls + nloc * 4) + 8 * (lane >> 5);
#pragma unroll
      for (int h = 0; h < 4; ++h) w[h] = *(const uint2*)(lb + 16 * (h ^ ((nloc >> 2) & 3)));
    }
    if (v0 + kTS <= a.V && all_rows) {  // uniform: nothing to mask
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t ww = (q & 3) < 2 ? w[q >> 2].x : w[q >> 2].y;
        acc[q] = (q & 1) ? bf16_hi(ww) : bf16_lo(ww);
      }
    } else {
      const int vb = v0 + 4 * (lane >> 5);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t ww = (q & 3) < 2 ? w[q >> 2].x : w[q >> 2].y;
        const bool ok = rvalid & (vb + 8 * (q >> 2) + (q & 3) < a.V);
        acc[q] = ok ? ((q & 1) ? bf16_hi(ww) : bf16_lo(ww)) : -INFINITY;
      }
    }
  };
  // epilogue of one stage for the log-sum-exp and sampled modes (z = acc)
  const float cz = MODE == MODE_SAMPLE ? a.cz : kLog2e;
  auto epilogue = [&](int s, const f32x16& zacc) {
    const int v0 = (s_begin + s) * kTS;
    f32x16 z = zacc;
    if (MODE == MODE_SAMPLE) {
      // round to bf16 (nearest, ties to even; infinities stay infinite), emit the row
      // entries of this stage (four runs of four consecutive tokens), and continue
      // with the rounded values
      uint32_t hb[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t u = __float_as_uint(z[q]);
        hb[q] = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
        z[q] = __uint_as_float(hb[q] << 16);
      }
      // through this wave's private LDS tile of a stage pair (32 rows x 64 tokens,
      // rows kZS bytes apart; the pair starts at an even global stage, so its 128
      // bytes per row are one aligned line): lanes write their runs of four into the
      // stage's half, and once the pair is complete (or the slice ends) read back 16
      // bytes each, so every global store writes 8 rows x 128 contiguous bytes. Halves
      // outside this slice (the first stage of a slice can be a pair's second half,
      // the last its first half) are not stored.
      char* zt = (char*)(lds + 2 * (WST + LST)) + wave * (32 * kZS);
      const int half = (s_begin + s) & 1;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint2 w;
        w.x = hb[4 * h] | (hb[4 * h + 1] << 16);
        w.y = hb[4 * h + 2] | (hb[4 * h + 3] << 16);
        *(uint2*)(zt + (lane & 31) * kZS + 64 * half + 16 * h + 8 * (lane >> 5)) = w;
      }
      if (half == 1 || s == nst - 1) {  // uniform over the workgroup
        const bool lo_ok = half == 0 || s >= 1;  // the pair's first stage belongs to this slice
        const bool hi_ok = half == 1;
        const int vp = v0 - 32 * half;            // the pair's first token
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rl = (lane >> 3) + 8 * j, ch = lane & 7;
          const uint4 w = *(const uint4*)(zt + rl * kZS + 16 * ch);
          const int grow = r0 + wave * 32 + rl;
          const int v = vp + 8 * ch;
          if (grow < a.rows && ((ch < 4) ? lo_ok : hi_ok)) {
            uint16_t* zp = a.zout + (size_t)grow * a.ldz_r + (size_t)a.d * a.ldz_d + v;
            if (v + 8 <= a.V) {
              *(uint4*)zp = w;
            } else {
              const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (v + e < a.V) zp[e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int v = v0 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      tmax = fmaxf(tmax, z[q]);
      if (MODE == MODE_ARGMAX_LSE && z[q] > best) {
        best = z[q];
        bidx = v;
      }
    }
    if (tmax != -INFINITY) {
      const float nref = fmaxf(lref, tmax * cz);
      float ts = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) ts += fast_exp2(__builtin_fmaf(z[q], cz, -nref));  // exp2(-inf) = 0
      const double scale = lref == -INFINITY ? 0.0 : (double)fast_exp2(lref - nref);
      lsum = lsum * scale + (double)ts;
      lref = nref;
    }
  };

  // Tree: the stage maximum tm and ts = sum of exp2(z log2e - lref) are accumulated one
  // value per MFMA of the next stage, against the reference of the stages before; then
  // the stage's end (reference update, top-4 insertion).
  auto tree_stage_end_s = [&](int s, const f32x16& z, float tm, float ts) {
    tree_stage_end((s_begin + s) * kTS, lane, z, tm, ts, lref, lsum, tv, ti, thr, th_row);
  };

  // Stages are software-pipelined inside each wave: the MFMAs of stage s are issued
  // first, then the epilogue of stage s-1 runs on the other accumulator (for the chain
  // and the tree, one value per MFMA, in program order between them).
  f32x16 acc[2];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[1][q] = -INFINITY;  // "stage -1": updates nothing
  for (int base = 0; base < nst; base += NU) {
#pragma unroll
    for (int p = 0; p < NU; ++p) {
      const int s = base + p;
      if (s >= nst) break;  // uniform over the workgroup
      const int b = p & 1;  // NU is even, so s & 1 == p & 1
      const int rp = p % NR;
      // stage s is the oldest of the NR stages in flight: wait for its loads only
      vm_wait<(NR - 1) * LPS>();
      if constexpr (AS) {  // what this wait covers: stage s of the ring (and, at s = 0, the U rows)
#pragma unroll
        for (int q = 0; q < WQ; ++q) landed(ringw[rp][q]);
#pragma unroll
        for (int q = 0; q < LQ; ++q) {
          if constexpr (LAL) {
            landed(ringl[rp][q]);
          } else {
#pragma unroll
            for (int l = 0; l < 8; ++l) landed(ringu[rp][q][l]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) landed(ufr[ks]);
      }
      // buffer b was last read two stages ago, before the previous barrier
      store_stage(b, ringw[rp], ringl[rp], ringu[rp]);
      __syncthreads();
      load_stage(s + NR, ringw[rp], ringl[rp], ringu[rp]);
      const u32x4* Ws = lds + b * (WST + LST);
      if (lk) {  // the base logits as the first k-step (accumulator from zero)
        const bf16x8 al = __builtin_bit_cast(
            bf16x8, *((const u32x4*)((const uint16_t*)(Ws + WST) + (lane & 31) * 16) + (lane >> 5)));
        f32x16 zero = {};
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, __builtin_bit_cast(bf16x8, onehot), zero, 0, 0, 0);
      } else {
        init_from_l(s, Ws + WST, acc[b]);
      }
      const int code0 = 16 * (s - 1);
      float tm = -INFINITY, ts = 0.f;  // tree: stage s-1 (discarded for s = 0)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int m = lane & 31, kv = 2 * ks + (lane >> 5);
        const bf16x8 af = __builtin_bit_cast(bf16x8, Ws[m * NV + swz_w(m, kv)]);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8, ufr[ks]), acc[b], 0, 0, 0);
        if (MODE == MODE_ARGMAX && ks < 16 && acc[b ^ 1][ks] > best) {
          best = acc[b ^ 1][ks];
          bcode = code0 + ks;
        }
        if (MODE == MODE_TREE && ks < 16) {
          tm = fmaxf(tm, acc[b ^ 1][ks]);
          ts += fast_exp2(__builtin_fmaf(acc[b ^ 1][ks], kLog2e, -lref));
        }
      }
      if (MODE == MODE_TREE) {
        if (lk) {  // tokens past V and rows past the block: -inf, as the per-row path starts them
          const int v0 = (s_begin + s) * kTS;
          if (!(v0 + kTS <= a.V && all_rows)) {  // uniform
            const int vb = v0 + 4 * (lane >> 5);
#pragma unroll
            for (int q = 0; q < 16; ++q)
              if (!(rvalid & (vb + 8 * (q >> 2) + (q & 3) < a.V))) acc[b][q] = -INFINITY;
          }
        }
#pragma unroll
        for (int q = KS; q < 16; ++q) {  // ranks below 256: the remaining values
          tm = fmaxf(tm, acc[b ^ 1][q]);
          ts += fast_exp2(__builtin_fmaf(acc[b ^ 1][q], kLog2e, -lref));
        }
        // s = 0: the stage before is the -inf sentinel, which changes nothing (its sum is
        // not selected, its maximum is -inf)
        tree_stage_end_s(s - 1, acc[b ^ 1], tm, ts);
      } else if (MODE == MODE_ARGMAX) {
#pragma unroll
        for (int q = KS; q < 16; ++q)  // ranks below 256: the remaining values
          if (acc[b ^ 1][q] > best) {
            best = acc[b ^ 1][q];
            bcode = code0 + q;
          }
      } else if (s > 0) {
        epilogue(s - 1, acc[b ^ 1]);
      }
    }
  }
  // The ring's trailing loads (past the range: they read zeros) must land before any
  // code after the loop runs: the ring registers are dead from here on, and the
  // compiler may hand them to the epilogue below while a load into them is in flight.
  vm_wait<0>();
  // the last stage's epilogue (accumulator picked by two static paths: indexing the
  // pair with a run-time value would move it to scratch memory)
  auto finish = [&](const f32x16& last) {
    if (MODE == MODE_ARGMAX) {
      const int code0 = 16 * (nst - 1);
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (last[q] > best) {
          best = last[q];
          bcode = code0 + q;
        }
    } else if (MODE == MODE_TREE) {
      float tm = -INFINITY, ts = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        tm = fmaxf(tm, last[q]);
        ts += fast_exp2(__builtin_fmaf(last[q], kLog2e, -lref));
      }
      tree_stage_end_s(nst - 1, last, tm, ts);
    } else {
      epilogue(nst - 1, last);
    }
  };
  if (nst > 0) {
    if ((nst - 1) & 1) finish(acc[1]);
    else finish(acc[0]);
  }
  if (MODE == MODE_ARGMAX && bcode >= 0) {
    const int q = bcode & 15;
    bidx = (s_begin + (bcode >> 4)) * kTS + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
  }

  // merge lane pairs (lane, lane ^ 32 hold the same parent row), then lanes < 32 write
  if (MODE == MODE_TREE) {
    merge_pair_top4(tv, ti);
  } else {
    const float ob = __shfl_xor(best, 32, 64);
    const int oi = __shfl_xor(bidx, 32, 64);
    if (ob > best || (ob == best && oi < bidx)) {
      best = ob;
      bidx = oi;
    }
  }
  if (MODE != MODE_ARGMAX) merge_pair_lse(lref, lsum);
  if (lane >= 32 || !rvalid) return;
  if (MODE == MODE_TREE) {
    TreePart p;
#pragma unroll
    for (int q = 0; q < kTopK; ++q) {
      p.val[q] = tv[q];
      p.idx[q] = ti[q];
    }
    p.ref = lref;
    p.pad = 0.f;
    p.sum = lsum;
    ((TreePart*)a.part)[(size_t)row * a.G + g] = p;
  } else {
    ChainPart p;
    p.key = bidx == 0x7fffffff ? 0ull : amax_key(best, (uint32_t)bidx);
    p.ref = lref;
    p.pad = 0.f;
    p.sum = MODE == MODE_ARGMAX ? 0.0 : lsum;
    ((ChainPart*)a.part)[(size_t)row * a.G + g] = p;
  }
}

// ---------------------------------------------------------------- tree GEMM, scheduled stages
// The tree's GEMM for row blocks spanning at most 16 requests (the PCTree's depths with
// a full frontier), at rank up to 256. Same workgroup shape, vocabulary slices, XCD
// grouping, partial results and arithmetic as markov_gemm_kernel's tree mode, with the
// base logits entering as the first k-step (A = the stage's 32 tokens x 16 requests of
// L, B = each row's one-hot request) and the k-steps summed in the same order, so z and
// every output are bit-identical to it. What differs is how a stage is issued:
//  - every streaming load goes straight from memory into LDS (buffer loads with the
//    lds modifier, issued from inline assembly so that no compiler-inserted wait drains
//    them): Wt stages and the L tile as stored, six stage slots, stages issued four
//    ahead. No register is the destination of a load in flight in the stage loop, so
//    the compiler cannot copy one before its wait; the stages go in pairs with one
//    barrier per pair. Each lane gathers its L fragment (8 requests of one token) from
//    the stored tile during the stage before.
//  - a fixed issue order per stage (scheduling barriers): Wt fragments read three
//    k-steps ahead of their MFMA, the previous stage's exp2 sums and maximum placed
//    between the MFMAs so they run while the matrix cores work, the stage's sum added
//    before the last MFMAs, and the next stages' loads spread over the k-steps instead
//    of issued by every wave at once after the barrier.
// A direct-to-LDS load of 16 bytes writes lane l's data at M0 + 16*l, so the swizzled
// Wt tile layout is made by choosing each lane's source address: slot t of a stage
// holds token row m = t / NV, swizzled vector p = t % NV, i.e. rank vector
// kv = swz(m, p) (the swizzle is an XOR, its own inverse).
__device__ __forceinline__ void dma_load_x4(uint32_t lds_addr, const s32x4& d, uint32_t off) {
  // s_nop 4: M0 is read by the load one instruction after it is written, and the
  // descriptor may come from a VALU write of an SGPR (5 wait states)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(off),
               "s"(d)
               : "memory");
}

template <int KS>
__global__ __launch_bounds__(kGT, 1) void tree_gemm_kernel(GemmArgs a) {
  static_assert(KS >= 2 && KS <= 16 && (KS & (KS - 1)) == 0, "rank up to 256");
  constexpr int NV = 2 * KS;                    // 16-byte vectors per staged Wt row
  constexpr int WST = kTS * NV;                 // Wt vectors per stage
  constexpr int WSLOT = WST > kGT ? WST : kGT;  // LDS vectors per Wt stage slot
  constexpr int WD = WSLOT / kGT;               // Wt direct-to-LDS loads per thread per stage
  constexpr int NS = 6;                         // stage slots (Wt and L): stage s in slot s % 6
  constexpr int LTV = kTS * 16 * 2 / 16;        // L tile vectors (16 requests x 32 tokens, bf16)
  extern __shared__ u32x4 lds[];                // [NS][WSLOT] Wt, then [NS][LTV] L tiles
  u32x4* const wbuf = lds;
  u32x4* const lbuf = lds + NS * WSLOT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int g, rb;
  {
    const int id = blockIdx.x;
    if (a.xcd_map) {
      const int j = id >> 3;
      g = (j / a.nrb) * 8 + (id & 7);
      rb = j % a.nrb;
    } else {
      g = id % a.G;
      rb = id / a.G;
    }
  }
  const int r0 = rb * kTR;
  const int nst_all = (a.V + kTS - 1) / kTS;
  const int s_begin = (int)(((long)g * nst_all) / a.G);
  const int nst = (int)(((long)(g + 1) * nst_all) / a.G) - s_begin;

  const int nloc = wave * 32 + (lane & 31);
  const int row = r0 + nloc;
  const bool rvalid = row < a.rows;
  const bool all_rows = r0 + kTR <= a.rows;
  int tok = 0;
  if (rvalid) {
    tok = a.row_tok[(size_t)row * a.ld_tok];
    if (tok < 0 || tok >= (a.u_rows > 0 ? a.u_rows : a.V)) {
      if (g == 0 && lane < 32) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
      tok = 0;
    }
  }
  u32x4 ufr[KS] = {};
  u32x4 onehot = {0u, 0u, 0u, 0u};
  if (rvalid) {
    const int j = row / a.rows_per_req - r0 / a.rows_per_req - 8 * (lane >> 5);
    if (j >= 0 && j < 8) onehot[j >> 1] = 0x3f80u << (16 * (j & 1));
  }

  const s32x4 wdesc = make_desc(a.Wt, (uint32_t)((size_t)a.V * a.rank * 2));
  const int req0 = r0 / a.rows_per_req;
  const int rlast = (r0 + kTR < a.rows ? r0 + kTR : a.rows) - 1;
  const int nreq = rlast / a.rows_per_req - req0 + 1;  // at most 16 (checked on the host)
  // the L rows of the block's requests (a 16-byte load ending past V reads the dword
  // holding V-1 whole: the extent is rounded up to it, still inside the row's storage)
  const s32x4 ldesc = make_desc(a.L + (size_t)req0 * a.ldL_r + (size_t)a.d * a.ldL_d,
                                (uint32_t)((((size_t)(nreq - 1) * a.ldL_r + a.V) * 2 + 3) & ~(size_t)3));
  // Wt: this thread's source offsets, less the stage term
  uint32_t wofs[WD];
#pragma unroll
  for (int q = 0; q < WD; ++q) {
    const int t = q * kGT + tid;
    const int m = t / NV, p = t % NV;
    constexpr int W = NV < 16 ? NV : 16, RW = 16 / W;
    const int kv = (p & ~(W - 1)) | ((p ^ (m / RW)) & (W - 1));
    wofs[q] = t < WST && kv * 8 < a.rank ? (uint32_t)((m * a.rank + kv * 8) * 2) : kOOB;
  }
  const uint32_t lds_w = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)wbuf;
  const uint32_t lds_l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)lbuf;
  // L (the first wave): lane l loads 8 tokens (16 bytes) of request l / 4, column l % 4,
  // into the tile [request][32 tokens] as stored (zero past the block's requests)
  const uint32_t lofs =
      lane >> 2 < nreq ? (uint32_t)(((size_t)(lane >> 2) * a.ldL_r + 8 * (lane & 3)) * 2) : kOOB;
  auto load_l = [&](int s) {
    if (wave == 0)  // uniform; the other waves' counted waits leave this load out
      dma_load_x4(lds_l + (uint32_t)((s % NS) * LTV * 16), ldesc,
                  lofs + (s < nst ? (uint32_t)((size_t)(s_begin + s) * kTS * 2) : kOOB));
  };
  auto load_w = [&](int s, int q) {
    const uint32_t tw = s < nst ? (uint32_t)((size_t)(s_begin + s) * kTS * a.rank * 2) : kOOB;
    const uint32_t slot = lds_w + (uint32_t)((s % NS) * WSLOT * 16);
    dma_load_x4(__builtin_amdgcn_readfirstlane(slot + (uint32_t)((q * kGT + wave * 64) * 16)), wdesc, wofs[q] + tw);
  };
  // the L k-step's A fragment of stage s: lane l holds token l % 32 of requests
  // 8*(l/32) .. +8, gathered from the stored tile. A non-finite entry is taken as -max
  // (a zero weight times an infinity would make NaN in every other request's sum): for a
  // masked -inf that ranks and weighs the same; +inf and NaN are faults, noted here and
  // reported once at the end (no branch in the stage loop).
  bool lfault = false;
  auto l_frag = [&](int s) {
    const uint16_t* t = (const uint16_t*)(lbuf + (s % NS) * LTV) + 8 * (lane >> 5) * kTS + (lane & 31);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = t[e * kTS];
    u32x4 v;
    // any non-finite entry: adding 0x80 to a bf16 exponent field (bits 7..14) carries into
    // bit 15 only when the field is all ones, and with both halves of a pair at once no
    // carry crosses into the upper half
    uint32_t any = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] = h[2 * c] | (h[2 * c + 1] << 16);
      any |= (v[c] & 0x7f807f80u) + 0x00800080u;
    }
    if (any & 0x80008000u) {  // rare: stage the non-finite entries
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool nonfinite = (h[e] & 0x7f80u) == 0x7f80u;
        lfault |= nonfinite & ((h[e] & 0x807fu) != 0x8000u);  // +inf or NaN
        h[e] = nonfinite ? 0xff7fu : h[e];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = h[2 * c] | (h[2 * c + 1] << 16);
    }
    return v;
  };

  float tv[kTopK];
  int ti[kTopK];
#pragma unroll
  for (int q = 0; q < kTopK; ++q) {
    tv[q] = -INFINITY;
    ti[q] = 0x7fffffff;
  }
  float lref = -INFINITY;
  double lsum = 0.0;
  float th_row = -INFINITY;
  if (a.theta && rvalid) th_row = a.theta[row];
  float thr = th_row;

  // Stages go in pairs (s, s + 1), s even, with one barrier per pair; every load goes
  // straight to LDS, so no register is written by a load in flight. Loads per pair, in
  // this order: the L tiles of stages s + 4 and s + 5 (first wave), then their Wt parts.
  // The wait at a pair's start leaves only the previous pair's Wt parts in flight, so
  // stages s and s + 1 (and the U rows) and the L tiles of s + 2 and s + 3 have landed.
  // A stage's slot is refilled (s + 4, s + 5) once its reads are before the barrier
  // (s - 2, s - 1); stage t's L fragment is gathered during stage t - 1.
  load_l(0);
  load_l(1);
#pragma unroll
  for (int q = 0; q < WD; ++q) load_w(0, q);
#pragma unroll
  for (int q = 0; q < WD; ++q) load_w(1, q);
  {
    const s32x4 udesc = make_desc(a.U, (uint32_t)((size_t)(a.u_rows > 0 ? a.u_rows : a.V) * a.rank * 2));
    const uint32_t ubase = (uint32_t)(((size_t)tok * a.rank + 8 * (lane >> 5)) * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool ok = rvalid && 16 * ks + 8 * (lane >> 5) < a.rank;
      buf_load_x4<true>(ufr[ks], udesc, ok ? ubase + 32 * ks : kOOB);
    }
  }
  load_l(2);
  load_l(3);
#pragma unroll
  for (int q = 0; q < WD; ++q) load_w(2, q);
#pragma unroll
  for (int q = 0; q < WD; ++q) load_w(3, q);
  // stage 0's L tile, for its fragment
  if (wave == 0) vm_wait<2 * WD + KS + 2 + 2 * WD>();
  __syncthreads();
  u32x4 alf = l_frag(0);

  // tokens past V and rows past the block are -inf (their L entries may hold another
  // request's logits); the masked values replace the stage's sums
  auto mask_stage = [&](int s, f32x16& z, float& tm, float& ts) {
    const int v0 = (s_begin + s) * kTS;
    const int vb = v0 + 4 * (lane >> 5);
    tm = -INFINITY;
    ts = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (!(rvalid & (vb + 8 * (q >> 2) + (q & 3) < a.V))) z[q] = -INFINITY;
      tm = fmaxf(tm, z[q]);
      ts += fast_exp2(__builtin_fmaf(z[q], kLog2e, -lref));
    }
  };

  // acc[b]: stage s (b = s & 1), the L k-step first and then every k-step in order, so z
  // is summed exactly as in markov_gemm_kernel; acc[b ^ 1] holds stage s - 1 for the epilogue
  f32x16 acc[2];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[1][q] = -INFINITY;  // "stage -1": updates nothing
  auto stage = [&](const int p, const int s) {
    const int b = p & 1;
    const u32x4* Ws = wbuf + p * WSLOT;  // s % NS (base is a multiple of NS)
    auto wfrag = [&](int ks) {
      const int m = lane & 31, kv = 2 * ks + (lane >> 5);
      constexpr int W = NV < 16 ? NV : 16, RW = 16 / W;
      return __builtin_bit_cast(bf16x8, Ws[m * NV + ((kv & ~(W - 1)) | ((kv ^ (m / RW)) & (W - 1)))]);
    };
    const f32x16 zero = {};
    const f32x16& z = acc[b ^ 1];  // stage s - 1
    const int v0p = (s_begin + s - 1) * kTS;
    // stage s - 1 needs the mask (tokens past V, rows past the block): then its sums are
    // taken again after the mask, and the in-section sum is not added
    const bool masked = !(v0p + kTS <= a.V && all_rows);  // uniform
    float tm = -INFINITY, ts = 0.f;
    bool fast = false;
    // Issue order, fixed by scheduling barriers, one group per k-step after its MFMA:
    // the Wt fragments are read three k-steps ahead (an MFMA never waits for its own
    // read); the 16 values of stage s - 1's epilogue run in the first VS groups and its
    // sum is added in the next, so no dependent chain trails the last MFMA; the next
    // stage's L fragment is gathered and stage s + 4's loads issued, spread over the
    // groups rather than queued by all waves at once after the barrier.
    constexpr int VS = KS >= 8 ? KS * 3 / 4 : KS;
    auto values = [&](int j) {
#pragma unroll
      for (int q = 16 * j / VS; q < 16 * (j + 1) / VS; ++q) {
        tm = fmaxf(tm, z[q]);
        ts += fast_exp2(__builtin_fmaf(z[q], kLog2e, -lref));
      }
    };
    bf16x8 fr[3];
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < KS) fr[j] = wfrag(j);
    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, alf), __builtin_bit_cast(bf16x8, onehot),
                                                     zero, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks % 3], __builtin_bit_cast(bf16x8, ufr[ks]), acc[b], 0, 0,
                                                       0);
      if (ks + 3 < KS) fr[ks % 3] = wfrag(ks + 3);
      if (ks < VS) values(ks);
      // (a stage to be masked adds nothing here: a -inf reference selects no sum)
      if (VS < KS && ks == VS) fast = tree_stage_sum(tm, ts, masked ? -INFINITY : lref, lsum);
      if (ks == 1) alf = l_frag(s + 1);  // stage s + 1's tile: landed before this pair's barrier or the last
      if (b == 0 && ks == 0) {
        load_l(s + 4);
        load_l(s + 5);
      }
#pragma unroll
      for (int q = 0; q < WD; ++q)
        if (ks == (KS * (q + 1)) / (WD + 1)) load_w(s + 4, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (VS == KS) fast = tree_stage_sum(tm, ts, masked ? -INFINITY : lref, lsum);
    // s = 0: the -inf sentinel, which changes nothing
    if (masked) {
      f32x16 zm = z;
      mask_stage(s - 1, zm, tm, ts);
      tree_stage_end(v0p, lane, zm, tm, ts, lref, lsum, tv, ti, thr, th_row);
    } else {
      tree_stage_rest(fast, v0p, lane, z, tm, lref, lsum, tv, ti, thr, th_row);
    }
  };
  for (int base = 0; base < nst; base += NS) {
#pragma unroll
    for (int p = 0; p < NS; p += 2) {
      const int s = base + p;
      if (s >= nst) break;  // uniform over the workgroup
      vm_wait<2 * WD>();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) landed(ufr[ks]);
      __syncthreads();
      stage(p, s);
      if (s + 1 < nst) {
        stage(p + 1, s + 1);
      } else {  // the pair's load count: stage s + 5's Wt parts (past the range)
#pragma unroll
        for (int q = 0; q < WD; ++q) load_w(s + 5, q);
      }
    }
  }
  vm_wait<0>();  // the trailing loads (past the range) land before the LDS is left
  auto finish = [&](const f32x16& last) {
    f32x16 z = last;
    float tm = -INFINITY, ts = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      tm = fmaxf(tm, z[q]);
      ts += fast_exp2(__builtin_fmaf(z[q], kLog2e, -lref));
    }
    const int v0 = (s_begin + nst - 1) * kTS;
    if (!(v0 + kTS <= a.V && all_rows)) mask_stage(nst - 1, z, tm, ts);
    tree_stage_end(v0, lane, z, tm, ts, lref, lsum, tv, ti, thr, th_row);
  };
  if (nst > 0) {
    if ((nst - 1) & 1) finish(acc[1]);
    else finish(acc[0]);
  }
  if (lfault) atomicOr(a.status, DSP_STATUS_NONFINITE);
  merge_pair_top4(tv, ti);
  merge_pair_lse(lref, lsum);
  if (lane >= 32 || !rvalid) return;
  TreePart p;
#pragma unroll
  for (int q = 0; q < kTopK; ++q) {
    p.val[q] = tv[q];
    p.idx[q] = ti[q];
  }
  p.ref = lref;
  p.pad = 0.f;
  p.sum = lsum;
  ((TreePart*)a.part)[(size_t)row * a.G + g] = p;
}

// ---------------------------------------------------------------- chain GEMM, scheduled stages
// The greedy chain's GEMM (arg-max only) for 16-byte aligned row-major L, at rank up to
// 256: the same workgroup shape, vocabulary slices, accumulators started from L and
// k-steps summed in order as markov_gemm_kernel's arg-max mode, so z, the arg-max and
// the partial results are bit-identical to it. The stage issue follows tree_gemm_kernel:
// Wt and L stages go straight from memory into LDS (direct-to-LDS buffer loads from
// inline assembly: no load in flight into a register inside the stage loop), four stage
// slots with three stages in flight, a stage's data waited one stage before its use so
// each lane reads its L entries for the next stage ahead of time; per k-step, fixed by
// scheduling barriers, the MFMA, the fragment read three k-steps ahead, one value of the
// previous stage's arg-max, and the next stages' loads spread over the k-steps.
template <int KS>
__global__ __launch_bounds__(kGT, 1) void chain_gemm_kernel(GemmArgs a) {
  static_assert(KS >= 2 && KS <= 16 && (KS & (KS - 1)) == 0, "rank up to 256");
  constexpr int NV = 2 * KS;                    // 16-byte vectors per staged Wt row
  constexpr int WST = kTS * NV;                 // Wt vectors per stage
  constexpr int WSLOT = WST > kGT ? WST : kGT;  // LDS vectors per Wt stage slot
  constexpr int WD = WSLOT / kGT;               // Wt loads per thread per stage
  constexpr int LST = kTR * 4;                  // L vectors per stage: 256 rows x 32 tokens
  constexpr int LD = LST / kGT;                 // L loads per thread per stage
  constexpr int LPS = WD + LD;                  // loads per stage per thread
  constexpr int NS = 4;                         // stage slots: stage s in slot s % 4
  extern __shared__ u32x4 lds[];                // [NS][WSLOT] Wt, then [NS][LST] L
  u32x4* const wbuf = lds;
  u32x4* const lbuf = lds + NS * WSLOT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int g, rb;
  {
    const int id = blockIdx.x;
    if (a.xcd_map) {
      const int j = id >> 3;
      g = (j / a.nrb) * 8 + (id & 7);
      rb = j % a.nrb;
    } else {
      g = id % a.G;
      rb = id / a.G;
    }
  }
  const int r0 = rb * kTR;
  const int nst_all = (a.V + kTS - 1) / kTS;
  const int s_begin = (int)(((long)g * nst_all) / a.G);
  const int nst = (int)(((long)(g + 1) * nst_all) / a.G) - s_begin;

  const int nloc = wave * 32 + (lane & 31);
  const int row = r0 + nloc;
  const bool rvalid = row < a.rows;
  const bool all_rows = r0 + kTR <= a.rows;
  int tok = 0;
  if (rvalid) {
    tok = a.row_tok[(size_t)row * a.ld_tok];
    if (tok < 0 || tok >= (a.u_rows > 0 ? a.u_rows : a.V)) {
      if (g == 0 && lane < 32) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
      tok = 0;
    }
  }
  u32x4 ufr[KS] = {};

  const s32x4 wdesc = make_desc(a.Wt, (uint32_t)((size_t)a.V * a.rank * 2));
  const int req0 = r0 / a.rows_per_req;
  const int rlast = (r0 + kTR < a.rows ? r0 + kTR : a.rows) - 1;
  // up to the block's last row's token V-1; a 16-byte load ending past it reads the dword
  // holding V-1 whole (the extent is rounded up to it, inside the row's storage)
  const s32x4 ldesc = make_desc(a.L + (size_t)req0 * a.ldL_r + (size_t)a.d * a.ldL_d,
                                (uint32_t)((((size_t)(rlast / a.rows_per_req - req0) * a.ldL_r + a.V) * 2 + 3) &
                                           ~(size_t)3));
  constexpr int W = NV < 16 ? NV : 16, RW = 16 / W;  // Wt tile swizzle (an XOR: its own inverse)
  uint32_t wofs[WD], lofs[LD];
#pragma unroll
  for (int q = 0; q < WD; ++q) {
    const int t = q * kGT + tid;
    const int m = t / NV, p = t % NV;
    const int kv = (p & ~(W - 1)) | ((p ^ (m / RW)) & (W - 1));
    wofs[q] = t < WST && kv * 8 < a.rank ? (uint32_t)((m * a.rank + kv * 8) * 2) : kOOB;
  }
  // L tile: row n holds 4 vectors of 8 tokens, vector c at n*4 + (c ^ ((n >> 2) & 3)), so the
  // 8-byte reads of 16 consecutive rows hit 16 distinct slots; slot t = n*4 + c' holds
  // vector c = c' ^ ((n >> 2) & 3) of row n
#pragma unroll
  for (int q = 0; q < LD; ++q) {
    const int t = q * kGT + tid;
    const int n = t >> 2, c = (t & 3) ^ ((n >> 2) & 3);
    lofs[q] = r0 + n < a.rows ? (uint32_t)((((size_t)(r0 + n) / a.rows_per_req - req0) * a.ldL_r + 8 * c) * 2) : kOOB;
  }
  const uint32_t lds_w = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)wbuf;
  const uint32_t lds_l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)lbuf;
  auto load_w = [&](int s, int q) {
    const uint32_t tw = s < nst ? (uint32_t)((size_t)(s_begin + s) * kTS * a.rank * 2) : kOOB;
    dma_load_x4(__builtin_amdgcn_readfirstlane(lds_w + (uint32_t)(((s % NS) * WSLOT + q * kGT + wave * 64) * 16)), wdesc,
                wofs[q] + tw);
  };
  auto load_l = [&](int s, int q) {
    const uint32_t tl = s < nst ? (uint32_t)((size_t)(s_begin + s) * kTS * 2) : kOOB;
    dma_load_x4(__builtin_amdgcn_readfirstlane(lds_l + (uint32_t)(((s % NS) * LST + q * kGT + wave * 64) * 16)), ldesc,
                lofs[q] + tl);
  };
  auto load_stage = [&](int s) {
#pragma unroll
    for (int q = 0; q < WD; ++q) load_w(s, q);
#pragma unroll
    for (int q = 0; q < LD; ++q) load_l(s, q);
  };
  // this lane's 16 L entries of stage s (token v0 + 8*(q>>2) + 4*(lane>>5) + (q&3) at value q)
  auto read_l = [&](int s, uint2 (&w)[4]) {
    const char* lb = (const char*)(lbuf + (s % NS) * LST + nloc * 4) + 8 * (lane >> 5);
#pragma unroll
    for (int h = 0; h < 4; ++h) w[h] = *(const uint2*)(lb + 16 * (h ^ ((nloc >> 2) & 3)));
  };

  float best = -INFINITY;
  int bcode = -1;  // 16 * stage + value index of best

  // Prologue: stage 0, the U rows, stages 1 and 2; stage 0's L entries once it landed.
  load_stage(0);
  {
    const s32x4 udesc = make_desc(a.U, (uint32_t)((size_t)(a.u_rows > 0 ? a.u_rows : a.V) * a.rank * 2));
    const uint32_t ubase = (uint32_t)(((size_t)tok * a.rank + 8 * (lane >> 5)) * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool ok = rvalid && 16 * ks + 8 * (lane >> 5) < a.rank;
      buf_load_x4<true>(ufr[ks], udesc, ok ? ubase + 32 * ks : kOOB);
    }
  }
  load_stage(1);
  load_stage(2);
  vm_wait<KS + 2 * LPS>();
  __syncthreads();
  uint2 lw[4];
  read_l(0, lw);

  f32x16 acc[2];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[1][q] = -INFINITY;  // "stage -1": updates nothing
  // stage s: at its start stage s + 1 has landed (each thread its own loads, then the
  // barrier), so its L entries are read during stage s; stage s + 3's loads go into the
  // slot of stage s - 1, read before this stage's barrier
  auto stage = [&](const int p, const int s) {
    const int b = p & 1;
    const u32x4* Ws = wbuf + p * WSLOT;  // s % NS (base is a multiple of NS)
    auto wfrag = [&](int ks) {
      const int m = lane & 31, kv = 2 * ks + (lane >> 5);
      return __builtin_bit_cast(bf16x8, Ws[m * NV + ((kv & ~(W - 1)) | ((kv ^ (m / RW)) & (W - 1)))]);
    };
    // the accumulators start from L (-inf for a token past V or a row past the block)
    const int v0 = (s_begin + s) * kTS;
    if (v0 + kTS <= a.V && all_rows) {  // uniform: nothing to mask
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t ww = (q & 3) < 2 ? lw[q >> 2].x : lw[q >> 2].y;
        acc[b][q] = (q & 1) ? bf16_hi(ww) : bf16_lo(ww);
      }
    } else {
      const int vb = v0 + 4 * (lane >> 5);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t ww = (q & 3) < 2 ? lw[q >> 2].x : lw[q >> 2].y;
        const bool ok = rvalid & (vb + 8 * (q >> 2) + (q & 3) < a.V);
        acc[b][q] = ok ? ((q & 1) ? bf16_hi(ww) : bf16_lo(ww)) : -INFINITY;
      }
    }
    const f32x16& z = acc[b ^ 1];  // stage s - 1
    const int code0 = 16 * (s - 1);
    constexpr int VPM = 16 / KS;
    bf16x8 fr[3];
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < KS) fr[j] = wfrag(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks % 3], __builtin_bit_cast(bf16x8, ufr[ks]), acc[b], 0, 0,
                                                       0);
      if (ks + 3 < KS) fr[ks % 3] = wfrag(ks + 3);
#pragma unroll
      for (int q = ks * VPM; q < (ks + 1) * VPM; ++q) {  // values in token order: ties keep the first
        const bool gt = z[q] > best;
        best = gt ? z[q] : best;
        bcode = gt ? code0 + q : bcode;
      }
      if (ks == 1) read_l(s + 1, lw);
#pragma unroll
      for (int q = 0; q < WD; ++q)
        if (ks == (KS * (q + 1)) / (LPS + 1)) load_w(s + 3, q);
#pragma unroll
      for (int q = 0; q < LD; ++q)
        if (ks == (KS * (WD + q + 1)) / (LPS + 1)) load_l(s + 3, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int base = 0; base < nst; base += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const int s = base + p;
      if (s >= nst) break;  // uniform over the workgroup
      vm_wait<LPS>();       // stage s + 1 landed: stage s + 2's loads may still be in flight
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) landed(ufr[ks]);
      __syncthreads();
      stage(p, s);
    }
  }
  vm_wait<0>();  // the trailing loads (past the range) land before the LDS is left
  auto finish = [&](const f32x16& last) {
    const int code0 = 16 * (nst - 1);
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (last[q] > best) {
        best = last[q];
        bcode = code0 + q;
      }
  };
  if (nst > 0) {
    if ((nst - 1) & 1) finish(acc[1]);
    else finish(acc[0]);
  }
  int bidx = 0x7fffffff;
  if (bcode >= 0) {
    const int q = bcode & 15;
    bidx = (s_begin + (bcode >> 4)) * kTS + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
  }
  const float ob = __shfl_xor(best, 32, 64);
  const int oi = __shfl_xor(bidx, 32, 64);
  if (ob > best || (ob == best && oi < bidx)) {
    best = ob;
    bidx = oi;
  }
  if (lane >= 32 || !rvalid) return;
  ChainPart pp;
  pp.key = bidx == 0x7fffffff ? 0ull : amax_key(best, (uint32_t)bidx);
  pp.ref = -INFINITY;
  pp.pad = 0.f;
  pp.sum = 0.0;
  ((ChainPart*)a.part)[(size_t)row * a.G + g] = pp;
}

// ---------------------------------------------------------------- chain merge
struct ChainMergeArgs {
  const ChainPart* part;
  int32_t G, R, d;
  int32_t* y;
  int64_t ld_y;
  float* logq;
};

// One wavefront per (row r, step a.d + blockIdx.y); the partials of step a.d + y start
// y * R * G entries after a.part.
__global__ __launch_bounds__(64) void chain_merge_kernel(ChainMergeArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const ChainPart* pr = a.part + ((size_t)blockIdx.y * a.R + r) * a.G;
  a.d += blockIdx.y;
  // G <= 256: at most four partials per lane, all loaded before any is used (clamped
  // index, masked after)
  ChainPart cp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cp[q] = pr[min(lane + 64 * q, a.G - 1)];
  uint64_t best = 0;
  float H = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane + 64 * q < a.G) {
      best = cp[q].key > best ? cp[q].key : best;
      H = fmaxf(H, cp[q].ref);
    }
  best = wave_max(best);
  if (lane == 0) a.y[(size_t)r * a.ld_y + a.d] = (int32_t)amax_index(best);
  if (a.logq) {
    H = wave_max(H);
    double S = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q < a.G && cp[q].ref != -INFINITY) S += cp[q].sum * exp2((double)cp[q].ref - (double)H);
    S = wave_sum(S);
    if (lane == 0) {
      const double lse2 = (double)H + log2(S);
      const double zy = (double)amax_value(best);
      a.logq[(size_t)r * a.ld_y + a.d] = (float)((zy * kLog2ed - lse2) * kLn2d);
    }
  }
}

// ---------------------------------------------------------------- persistent greedy chain
// All steps of the greedy chain in one launch, one workgroup per CU. Between steps the
// chain needs every row's arg-max over the whole vocabulary before any row can fetch its
// next U row, so the steps are separated by a grid-wide barrier; what the barrier buys
// is that each workgroup keeps ITS vocabulary slice of Wt on chip for all the steps
// (rank 256: 16 KB per 32-token tile; up to 19 tiles per workgroup, 3 per wave in
// registers and the rest in LDS), so a step streams only the base logits L (and 256
// U rows from L2) instead of L plus all of Wt.
//
// Workgroup: 4 waves (one per SIMD, up to 512 registers each). Wave w owns a contiguous
// run of at most 5 tiles of the workgroup's slice and computes them for every parent row,
// one 32-row column block at a time: the column block's U rows are staged in LDS (double
// buffered, fetched during the block before) and read once as the 16 B fragments of
// the block; each tile then takes 16 MFMAs with its Wt fragments from registers or LDS.
// Tiles hold the Wt rows in the order tmap(i), so that the 16 accumulators of a lane are
// 16 consecutive tokens of its row and its L values are two 16-byte loads (row-major L).
// The arg-max (and log-sum-exp) per row is combined over lanes and waves in LDS, then
// over workgroups by a 64-bit atomic max of the order key (value, lowest id) into one of
// 8 copies per row, so that each copy takes the atomics of an eighth of the workgroups;
// the next step's tokens are the maxima of the 8 copies. The per-workgroup partials also
// go to the workspace, from which a merge kernel writes y and log q after the launch.
//
// The barrier is a counter that every workgroup raises once per step and then polls.
// It needs every workgroup resident at once (one per CU, which the launch shape and the
// resource use guarantee on an idle device); the poll is bounded, and a workgroup that
// waits past the bound sets DSP_STATUS_TIMEOUT and leaves, so the launch always drains.
constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPRegTiles = 3;   // Wt tiles per wave in registers
constexpr int kPWaveTiles = 5;  // tiles per wave at most
constexpr int kPMaxTiles = 19;  // tiles per workgroup at most (5, 5, 5, 4)
constexpr int kPLdsSlots = 7;   // Wt tiles in LDS: waves 0..2 two each, wave 3 one
constexpr int kPMaxR = 256;     // parent rows
constexpr int kPGroups = 8;     // arg-max key copies per row
constexpr int kPKeyStride = 16;  // uint64 words between keys: one 128-byte line each, so the
                                 // atomics of a step spread over the memory channels
constexpr int kPRowVec = 33;                // 16-byte vectors per LDS tile row: 32 + 1 of padding
constexpr int kPTileVec = 32 * kPRowVec;     // per LDS tile (32 rows x 512 bytes, padded)
constexpr int kCachePolicySC1 = 16;          // buffer access cache policy: SC1 (device scope)

struct PMerge {  // a row's partial over some tiles
  float best;
  int32_t idx;
  float ref;
  float sum;  // of at most a workgroup's 608 terms, each at most 1
};
static_assert(sizeof(PMerge) == 16, "persistent merge record");
constexpr size_t kPOffU = (size_t)kPLdsSlots * kPTileVec * 16;
constexpr size_t kPOffM = kPOffU + (size_t)2 * kPTileVec * 16;
constexpr size_t kPOffP = kPOffM + (size_t)2 * kPWaves * 32 * sizeof(PMerge);
constexpr size_t kPOffT = kPOffP + (size_t)kPMaxR * sizeof(PMerge);
constexpr size_t kPOffF = kPOffT + (size_t)kPMaxR * 4;
constexpr size_t kPLds = kPOffF + 16;
static_assert(kPLds <= 160 * 1024, "persistent chain LDS");

struct PersistArgs {
  const uint16_t* U;
  const uint16_t* Wt;
  const uint16_t* L;
  int64_t ldL_r, ldL_d;
  const int32_t* prev_tok;
  int32_t V, R, n_steps, G;
  ChainPart* part;    // [n_steps][R][G]
  uint64_t* keys;     // [n_steps][kPGroups][R], zero on entry
  uint32_t* bar;      // zero on entry
  uint32_t spin_limit;
  int32_t* status;
};

// MFMA row i of a tile holds token tmap(i): with i = 8j + 4h + k the accumulator q = 4j + k
// of a lane in half h is token 16h + q.
__device__ __forceinline__ int ptmap(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }
// 16-byte slot of vector kv of row m in an LDS tile: rows are 33 slots apart, so the 16 rows
// read together by a quarter wavefront start 4 banks apart and cover all 64 banks, and the
// slots of one lane's 16 fragments are a fixed stride apart (instruction offsets).
__device__ __forceinline__ int pslot(int m, int kv) { return m * kPRowVec + kv; }

template <bool LSE>
__device__ __forceinline__ void pmerge(PMerge& a, const PMerge& b) {
  if (b.best > a.best || (b.best == a.best && b.idx < a.idx)) {
    a.best = b.best;
    a.idx = b.idx;
  }
  if (!LSE) return;
  const float nref = fmaxf(a.ref, b.ref);
  float s = 0.f;
  if (a.ref != -INFINITY) s += a.sum * fast_exp2(a.ref - nref);
  if (b.ref != -INFINITY) s += b.sum * fast_exp2(b.ref - nref);
  a.ref = nref;
  a.sum = s;
}

template <bool LSE>
__global__ __launch_bounds__(kPThreads, 1) void chain_persist_kernel(PersistArgs a) {
  extern __shared__ u32x4 plds[];
  u32x4* Wl = plds;
  u32x4* Ub = plds + kPOffU / 16;
  PMerge* Mg = (PMerge*)((char*)plds + kPOffM);
  PMerge* Pt = (PMerge*)((char*)plds + kPOffP);
  int32_t* Tk = (int32_t*)((char*)plds + kPOffT);
  int32_t* Fl = (int32_t*)((char*)plds + kPOffF);

  // the wave index as a scalar: what derives from it (this wave's tiles, their count) is
  // then scalar too, so the per-tile tests are scalar branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
            col = lane & 31;
  const int g = blockIdx.x, grp = g & (kPGroups - 1);
  const int V = a.V, R = a.R, nsteps = a.n_steps;
  const int nst_all = (V + 31) / 32;
  const int tb = (int)(((long)g * nst_all) / a.G);
  const int ng = (int)(((long)(g + 1) * nst_all) / a.G) - tb;
  // tiles of this wave (at most 5, and 4 for the last wave, which has one LDS slot: the
  // host keeps ng <= 19, and the clamp keeps every index inside the layout regardless)
  const int nw = min(ng / 4 + (wave < ng % 4 ? 1 : 0), wave == kPWaves - 1 ? kPWaveTiles - 1 : kPWaveTiles);
  const int tw = tb + wave * (ng / 4) + min(wave, ng % 4);  // this wave's first tile
  const int nc = (R + 31) / 32;

  const s32x4 wdesc = make_desc(a.Wt, (uint32_t)((size_t)V * 512));
  const s32x4 udesc = make_desc(a.U, (uint32_t)((size_t)V * 512));
  const s32x4 kdesc = make_desc(a.keys, (uint32_t)((size_t)nsteps * kPGroups * R * kPKeyStride * 8));
  // extent up to the last (row, step)'s token V-1, rounded up to the end of its dword (the
  // range check is per dword; the base is 16-byte aligned)
  const s32x4 ldesc = make_desc(
      a.L, (uint32_t)((((size_t)(R - 1) * a.ldL_r + (size_t)(nsteps - 1) * a.ldL_d + V) * 2 + 3) & ~(size_t)3));

  // parent tokens of step 0
  if (tid < R) {
    int t = a.prev_tok[tid];
    if (t < 0 || t >= V) {
      if (g == 0) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
      t = 0;
    }
    Tk[tid] = t;
  }
  // Wt tiles past the third of this wave: to its LDS slots (loaded through registers)
#pragma unroll
  for (int j = kPRegTiles; j < kPWaveTiles; ++j) {
    if (wave == kPWaves - 1 && j == kPWaveTiles - 1) continue;  // wave 3 has one slot
    const int slot = 2 * wave + (j - kPRegTiles);
    u32x4 tmp[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int e = lane + 64 * p, i = e >> 5, kv = e & 31;
      const int v = (tw + j) * 32 + ptmap(i);
      buf_load_x4<false>(tmp[p], wdesc, j < nw && v < V ? (uint32_t)(((size_t)v * 256 + 8 * kv) * 2) : kOOB);
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int e = lane + 64 * p;
      Wl[slot * kPTileVec + pslot(e >> 5, e & 31)] = tmp[p];
    }
  }
  __syncthreads();  // Tk

  // Wt tiles 0..2 of this wave in registers: fragment ks of tile j = the 16 bytes of rank
  // 16ks + 8h .. +8 of token tmap(col). These and the first fills of the L ring and the U
  // staging use the compiler's own loads (it waits for them before any use, including a
  // register copy); the loads inside the step loop are the asynchronous ones.
  u32x4 wr[kPRegTiles][16];
#pragma unroll
  for (int j = 0; j < kPRegTiles; ++j) {
    const int v = (tw + j) * 32 + ptmap(col);
    const bool ok = j < nw && v < V;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      buf_load_x4<false>(wr[j][ks], wdesc, ok ? (uint32_t)(((size_t)v * 256 + 8 * (2 * ks + h)) * 2) : kOOB);
  }
  // L ring: slot j holds tile j of the next (step, column block) this wave computes;
  // lane (col, h) loads tokens 16h .. 16h+15 of row 32c + col
  u32x4 ring[kPWaveTiles][2];
  // lane base of the wave's tiles in row 32c + col of step d (tile j at +64j bytes, the
  // second 16 bytes at +16: instruction offsets); past the steps or rows: kOOB, whose
  // offsets stay past every extent. A wave with fewer than 5 tiles still loads 5 (the
  // extra ones are never used), so every wave issues the same count.
  auto l_base = [&](int d, int c) -> uint32_t {
    const int r = c * 32 + col;
    if (d >= nsteps || r >= R) return kOOB;
    return (uint32_t)(((size_t)r * a.ldL_r + (size_t)d * a.ldL_d + (size_t)tw * 32 + 16 * h) * 2);
  };
  auto l_load = [&](auto jc, uint32_t base, bool async) {
    constexpr int j = decltype(jc)::value;
    if (async) {
      buf_load_x4<true, 64 * j>(ring[j][0], ldesc, base);
      buf_load_x4<true, 64 * j + 16>(ring[j][1], ldesc, base);
    } else {
      buf_load_x4<false, 64 * j>(ring[j][0], ldesc, base);
      buf_load_x4<false, 64 * j + 16>(ring[j][1], ldesc, base);
    }
  };
  {
    const uint32_t b0 = l_base(0, 0);
    l_load(std::integral_constant<int, 0>{}, b0, false);
    l_load(std::integral_constant<int, 1>{}, b0, false);
    l_load(std::integral_constant<int, 2>{}, b0, false);
    l_load(std::integral_constant<int, 3>{}, b0, false);
    l_load(std::integral_constant<int, 4>{}, b0, false);
  }
  // U rows of a column block: thread -> row tid/8, vectors 4*(tid%8) .. +4
  u32x4 ur[4];
  auto u_offset = [&](int c) -> uint32_t {  // vector e of the thread's four at +16e bytes
    const int r = c * 32 + (tid >> 3);
    if (c >= nc || r >= R) return kOOB;
    return (uint32_t)(((size_t)Tk[r] * 256 + 8 * 4 * (tid & 7)) * 2);
  };
  auto load_u = [&](int c) {
    const uint32_t o = u_offset(c);
    buf_load_x4<true, 0>(ur[0], udesc, o);
    buf_load_x4<true, 16>(ur[1], udesc, o);
    buf_load_x4<true, 32>(ur[2], udesc, o);
    buf_load_x4<true, 48>(ur[3], udesc, o);
  };
  // One dword of each 128-byte line of every parent row's U row (thread r takes row r):
  // the lines and their translations are then in L2 when the column blocks' U rows are
  // fetched one block ahead of their use, instead of each block paying a full memory round
  // trip behind the one before. Issued together with the first block's rows.
  uint32_t pf[4] = {0u, 0u, 0u, 0u};
  auto prefetch_u = [&]() {
    const bool ok = tid < R;
    const int t = ok ? Tk[tid] : 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) buf_load_x1<true>(pf[e], udesc, ok ? (uint32_t)((size_t)t * 512 + 128 * e) : kOOB);
  };
  auto store_u = [&](int buf) {
    const int j = tid >> 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) Ub[buf * kPTileVec + pslot(j, 4 * (tid & 7) + e)] = ur[e];
  };
  {
    const uint32_t o = u_offset(0);
    buf_load_x4<false, 0>(ur[0], udesc, o);
    buf_load_x4<false, 16>(ur[1], udesc, o);
    buf_load_x4<false, 32>(ur[2], udesc, o);
    buf_load_x4<false, 48>(ur[3], udesc, o);
  }
  prefetch_u();
  vm_wait<0>();
#pragma unroll
  for (int e = 0; e < 4; ++e) landed(pf[e]);
  // every value above is waited for here, before the step loop
  // the register tiles live in the accumulation registers (AGPRs), which the MFMAs read
  // as their A operand directly; the arch VGPRs stay for everything else
#pragma unroll
  for (int j = 0; j < kPRegTiles; ++j)
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(wr[j][ks]));
#pragma unroll
  for (int j = 0; j < kPWaveTiles; ++j) {
    landed(ring[j][0]);
    landed(ring[j][1]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) landed(ur[e]);
  store_u(0);
  __syncthreads();

  for (int d = 0; d < nsteps; ++d) {
    for (int c = 0; c < nc; ++c) {
      // this column block's U fragments (B operand): row col, rank 16ks + 8h .. +8
      u32x4 bf[16];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) bf[ks] = Ub[(c & 1) * kPTileVec + pslot(col, 2 * ks + h)];
      load_u(c + 1);  // OOB past the last block: zeros, and the wait counts stay fixed
      const int dn = c + 1 < nc ? d : d + 1, cn = c + 1 < nc ? c + 1 : 0;
      float best = -INFINITY, lref = -INFINITY;
      int bq = -1;
      double lsum = 0.0;
      auto epi_lse = [&](const f32x16& z) {
        float tmax = -INFINITY;
#pragma unroll
        for (int q = 0; q < 16; ++q) tmax = fmaxf(tmax, z[q]);
        if (tmax != -INFINITY) {
          const float nref = fmaxf(lref, tmax * kLog2e);
          float ts = 0.f;
#pragma unroll
          for (int q = 0; q < 16; ++q) ts += fast_exp2(__builtin_fmaf(z[q], kLog2e, -nref));
          const double scale = lref == -INFINITY ? 0.0 : (double)fast_exp2(lref - nref);
          lsum = lsum * scale + (double)ts;
          lref = nref;
        }
      };
      const uint32_t lnext = l_base(dn, cn);
      // The accumulator of tile j starts from its L values (-inf for a token past V, and
      // for every entry of a tile past this wave's count, whose Wt rows are zero): the
      // MFMAs then leave z itself, and such entries never win or weigh.
      auto init = [&](auto jc, f32x16& z) {
        constexpr int j = decltype(jc)::value;
        landed(ring[j][0]);
        landed(ring[j][1]);
        const int v0 = (tw + j) * 32;
        if (j < nw && v0 + 32 <= V) {  // uniform
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const uint32_t w = ring[j][q >> 3][(q & 7) >> 1];
            z[q] = (q & 1) ? bf16_hi(w) : bf16_lo(w);
          }
        } else {
          // entries left in this lane's run of the vocabulary (computed here, so that the
          // 16 comparisons are not hoisted out of the loops and held as masks)
          int left = j < nw ? V - v0 - 16 * h : 0;
          asm volatile("" : "+v"(left));
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const uint32_t w = ring[j][q >> 3][(q & 7) >> 1];
            const float f = (q & 1) ? bf16_hi(w) : bf16_lo(w);
            z[q] = q < left ? f : -INFINITY;
          }
        }
        l_load(jc, lnext, true);  // slot j: the same tile of the next (step, block)
      };
      auto wfrag = [&](auto jc, int ks) -> bf16x8 {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < kPRegTiles) return __builtin_bit_cast(bf16x8, wr[j][ks]);
        else return __builtin_bit_cast(bf16x8, Wl[(2 * wave + j - kPRegTiles) * kPTileVec + pslot(col, 2 * ks + h)]);
      };
      auto mfma = [&](const bf16x8& af, int ks, f32x16& z) {
        z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8, bf[ks]), z, 0, 0, 0);
      };
      auto arg = [&](float z, int code) {  // tokens visited in increasing order
        if (z > best) {
          best = z;
          bq = code;
        }
      };
      // Tiles go two at a time with their MFMA chains interleaved (each MFMA then waits on
      // the one issued two slots before it, not on its predecessor), and the arg-max of the
      // two tiles before runs between them, 2 values per k-step in token order.
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using I4 = std::integral_constant<int, 4>;
      f32x16 acc[4];
      // slots 0, 1: after them came slots 2..4 of the block before and this block's U rows
      vm_wait<2 * 3 + 4>();
      init(I0{}, acc[0]);
      init(I1{}, acc[1]);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        mfma(wfrag(I0{}, ks), ks, acc[0]);
        mfma(wfrag(I1{}, ks), ks, acc[1]);
      }
      // slots 2, 3: after them, slot 4 of the block before, the U rows, the refills of 0, 1
      vm_wait<2 + 4 + 4>();
      init(I2{}, acc[2]);
      init(I3{}, acc[3]);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        mfma(wfrag(I2{}, ks), ks, acc[2]);
        mfma(wfrag(I3{}, ks), ks, acc[3]);
        arg(ks < 8 ? acc[0][2 * ks] : acc[1][2 * ks - 16], 2 * ks);
        arg(ks < 8 ? acc[0][2 * ks + 1] : acc[1][2 * ks - 15], 2 * ks + 1);
      }
      // instruction order for the scheduler: the LDS-tile fragments are read two k-steps
      // ahead; per k-step, an MFMA, half of the step's arg-max work, the next read, the
      // other MFMA, the other half
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        if (ks < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      // the arg-max of tiles 0, 1 completes here (otherwise the compiler may sink it past
      // the next tiles' MFMAs, out of the slots between them)
      asm volatile("" : "+v"(best), "+v"(bq));
      if (LSE) {
        epi_lse(acc[0]);
        epi_lse(acc[1]);
      }
      // slot 4: after it, the U rows and the refills of 0..3
      vm_wait<4 + 8>();
      init(I4{}, acc[0]);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        mfma(wfrag(I4{}, ks), ks, acc[0]);
        arg(ks < 8 ? acc[2][2 * ks] : acc[3][2 * ks - 16], 32 + 2 * ks);
        arg(ks < 8 ? acc[2][2 * ks + 1] : acc[3][2 * ks - 15], 32 + 2 * ks + 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        if (ks < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      asm volatile("" : "+v"(best), "+v"(bq));
#pragma unroll
      for (int q = 0; q < 16; ++q) arg(acc[0][q], 64 + q);
      if (LSE) {
        epi_lse(acc[2]);
        epi_lse(acc[3]);
        epi_lse(acc[0]);
      }
      PMerge m;
      m.best = best;
      m.idx = bq < 0 ? 0x7fffffff : (tw + (bq >> 4)) * 32 + 16 * h + (bq & 15);
      m.ref = lref;
      m.sum = (float)lsum;
      {
        PMerge o;
        o.best = __shfl_xor(m.best, 32, 64);
        o.idx = __shfl_xor(m.idx, 32, 64);
        if (LSE) {
          o.ref = __shfl_xor(m.ref, 32, 64);
          o.sum = __shfl_xor(m.sum, 32, 64);
        }
        pmerge<LSE>(m, o);
      }
      if (lane < 32) Mg[((c & 1) * kPWaves + wave) * 32 + lane] = m;
      // the next column block's U rows: 10 ring loads were issued after them
      vm_wait<2 * kPWaveTiles>();
#pragma unroll
      for (int e = 0; e < 4; ++e) landed(ur[e]);
      if (c + 1 == nc) {
        // leaving the column loop: the ring (now the next step's first block) lands
        // here, so that any register copy the compiler places on the way out of the
        // loop copies loaded values (the key update below waits for it anyway)
        vm_wait<0>();
#pragma unroll
        for (int j = 0; j < kPWaveTiles; ++j) {
          landed(ring[j][0]);
          landed(ring[j][1]);
        }
      }
      if (c + 1 < nc) store_u((c + 1) & 1);
      __syncthreads();
      if (wave == 0 && lane < 32 && c * 32 + lane < R) {
        PMerge p = Mg[(c & 1) * kPWaves * 32 + lane];
#pragma unroll
        for (int w = 1; w < kPWaves; ++w) pmerge<LSE>(p, Mg[((c & 1) * kPWaves + w) * 32 + lane]);
        Pt[c * 32 + lane] = p;
      }
    }
    __syncthreads();  // Pt complete
    if (tid < R) {
      const PMerge p = Pt[tid];
      const uint64_t key = p.idx == 0x7fffffff ? 0ull : amax_key(p.best, (uint32_t)p.idx);
      __hip_atomic_fetch_max(a.keys + (((size_t)d * kPGroups + grp) * R + tid) * kPKeyStride, key,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (LSE) {  // log q needs every workgroup's log-sum-exp partial; y alone, the keys
        ChainPart cp;
        cp.key = key;
        cp.ref = p.ref;
        cp.pad = 0.f;
        cp.sum = (double)p.sum;
        a.part[((size_t)d * R + tid) * a.G + g] = cp;
      }
    }
    if (d + 1 == nsteps) break;
    // Every exchange between workgroups is an agent-scope atomic (the key updates, the
    // counter, the key and counter reads), performed and read at the device's coherence
    // point, so no cache write-back or invalidation is needed (fences here would write
    // back and invalidate the L2 of the XCD, per thread and per step). What is needed is
    // that this workgroup's key updates are performed before its arrival is counted: each
    // thread waits for its own (vmcnt 0), then the workgroup barrier orders them before
    // the arrival.
    vm_wait<0>();
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t target = (uint32_t)(d + 1) * (uint32_t)a.G;
      uint32_t polls = 0;
      int ok = 1;
      while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++polls > a.spin_limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      if (!ok) atomicOr(a.status, DSP_STATUS_TIMEOUT);
      Fl[0] = ok;
    }
    __syncthreads();
    if (!Fl[0]) return;  // uniform; every load issued so far has landed (wait above)
    if (tid < R) {
      // the 8 copies of the row's key, read at the device's coherence point (SC1: the
      // updates are atomics performed there) with plain loads, all issued before any
      // is waited for (one memory round trip, not eight)
      uint64_t kq[kPGroups];
#pragma unroll
      for (int q = 0; q < kPGroups; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(
            as_rsrc(kdesc), (uint32_t)((((size_t)d * kPGroups + q) * R + tid) * kPKeyStride * 8), 0,
            kCachePolicySC1);
        kq[q] = ((uint64_t)v[1] << 32) | v[0];
      }
      uint64_t k = 0;
#pragma unroll
      for (int q = 0; q < kPGroups; ++q) k = kq[q] > k ? kq[q] : k;
      int t = k == 0 ? -1 : (int)amax_index(k);
      if (t < 0 || t >= V) {  // no finite entry in the row: as the per-step path, U row 0
        if (g == 0) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
        t = 0;
      }
      Tk[tid] = t;
    }
    __syncthreads();
    load_u(0);
    prefetch_u();
    vm_wait<0>();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      landed(ur[e]);
      landed(pf[e]);
    }
#pragma unroll
    for (int j = 0; j < kPWaveTiles; ++j) {
      landed(ring[j][0]);
      landed(ring[j][1]);
    }
    store_u(0);
    __syncthreads();
  }
  vm_wait<0>();  // the last refills (past the range, zeros) land before the waves end
#pragma unroll
  for (int j = 0; j < kPWaveTiles; ++j) {
    landed(ring[j][0]);
    landed(ring[j][1]);
  }
}

struct PersistInitArgs {
  uint64_t* keys;
  size_t n_keys;  // keys (kPKeyStride words apart)
  uint32_t* bar;
};
__global__ __launch_bounds__(256) void chain_persist_init_kernel(PersistInitArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < a.n_keys) a.keys[i * kPKeyStride] = 0ull;
  if (i == 0) *a.bar = 0u;
}

// y of the greedy chain from the persistent launch's keys: row r, step d (one thread each)
struct PersistYArgs {
  const uint64_t* keys;
  int32_t R, n_steps;
  int32_t* y;
  int64_t ld_y;
};
__global__ __launch_bounds__(256) void chain_persist_y_kernel(PersistYArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.R * a.n_steps) return;
  const int d = i / a.R, r = i % a.R;
  uint64_t k = 0;
#pragma unroll
  for (int q = 0; q < kPGroups; ++q) {
    const uint64_t kq = a.keys[(((size_t)d * kPGroups + q) * a.R + r) * kPKeyStride];
    k = kq > k ? kq : k;
  }
  a.y[(size_t)r * a.ld_y + d] = (int32_t)amax_index(k);  // no finite entry: -1, as the merge
}

// ---------------------------------------------------------------- sampled chain draw
struct ChainSampleArgs {
  const ChainPart* part;  // [R][G] log-sum-exp partials of the rounded row per vocabulary slice
  int32_t G, R, d, V;
  const uint16_t* z;      // the emitted bf16 rows
  int64_t ldz_r, ldz_d;
  float cz;               // log2(e) / T
  uint64_t seed, round;
  const uint64_t* round_dev;
  const int64_t* req_id;
  int32_t* y;
  int64_t ld_y;
  float* logq;
  int32_t* status;
};

// Inclusive prefix sum over the wavefront (fixed Hillis-Steele order, fp64).
__device__ __forceinline__ double wave_scan_incl(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double w = __shfl_up(v, o, 64);
    if (lane >= o) v += w;
  }
  return v;
}

// Inverse-CDF draw of step d for row r, one wavefront per row: the vocabulary slices'
// masses (from the GEMM partials) locate the slice that holds u * total, then that
// slice of the emitted bf16 row is rescanned in ascending token order, lane by lane
// over contiguous ranges, to the first token whose running mass exceeds the target
// (the last token with mass if rounding leaves none). Slices are the GEMM's: slice g
// covers 32-token stages [g*nst/G, (g+1)*nst/G).
__global__ __launch_bounds__(64) void chain_sample_kernel(ChainSampleArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const ChainPart* pr = a.part + (size_t)r * a.G;
  const int gpl = (a.G + 63) / 64;  // slices per lane (G <= 256)
  float ref[4];
  double sum[4];
  // unconditional loads (clamped index, masked after): a load under a branch is
  // waited for on the spot
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = lane * gpl + q;
    const bool in = q < gpl && g < a.G;
    const ChainPart pg = pr[in ? g : a.G - 1];
    ref[q] = in ? pg.ref : -INFINITY;
    sum[q] = in ? pg.sum : 0.0;
  }
  float H = fmaxf(fmaxf(ref[0], ref[1]), fmaxf(ref[2], ref[3]));
  H = wave_max(H);
  double w[4], lsum = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = ref[q] == -INFINITY ? 0.0 : sum[q] * (double)fast_exp2(ref[q] - H);
    lsum += w[q];
  }
  const double incl = wave_scan_incl(lsum);
  const double total = __shfl(incl, 63, 64);
  int32_t* yo = a.y + (size_t)r * a.ld_y + a.d;
  if (!(total > 0.0) || !(H < INFINITY) || total == INFINITY) {
    if (lane == 0) {
      *yo = -1;
      if (a.logq) a.logq[(size_t)r * a.ld_y + a.d] = NAN;
      atomicOr(a.status, DSP_STATUS_NONFINITE);
    }
    return;
  }
  const uint64_t rid = a.req_id ? (uint64_t)a.req_id[r] : (uint64_t)r;
  const uint64_t rnd = a.round_dev ? *a.round_dev : a.round;
  uint64_t c[4] = {rnd, rid, (uint64_t)(a.d + 1), 1ull};  // stream 1: the draft's draws
  philox4x64_10(c, a.seed, 0ull);
  const double tau = unit_double(c[0]) * total;
  // the slice holding tau (else the last slice with mass)
  const double excl = incl - lsum;
  const uint64_t hit = __ballot(lsum > 0.0 && excl <= tau && tau < incl);
  int gs = -1;
  double tin = INFINITY;  // target inside the slice; +inf: take its last token with mass
  if (hit) {
    const int l = __ffsll((unsigned long long)hit) - 1;
    if (lane == l) {
      double acc = excl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (gs < 0 && w[q] > 0.0 && tau < acc + w[q]) {
          gs = lane * gpl + q;
          tin = tau - acc;
        }
        acc += w[q];
      }
      if (gs < 0) {  // rounding between the per-slice and the lane sums: last slice with mass
        for (int q = 3; q >= 0; --q)
          if (gs < 0 && w[q] > 0.0) gs = lane * gpl + q;
      }
    }
    gs = __shfl(gs, l, 64);
    tin = __shfl(tin, l, 64);
  } else {
    const uint64_t any = __ballot(lsum > 0.0);
    const int l = 63 - __clzll((long long)any);
    if (lane == l)
      for (int q = 3; q >= 0; --q)
        if (gs < 0 && w[q] > 0.0) gs = lane * gpl + q;
    gs = __shfl(gs, l, 64);
  }
  const int nst_all = (a.V + 31) / 32;
  const int t0 = (int)(((long)gs * nst_all) / a.G) * 32;
  const int t1 = min(a.V, (int)(((long)(gs + 1) * nst_all) / a.G) * 32);
  const int per = (t1 - t0 + 63) / 64;
  const int v0 = min(t1, t0 + lane * per), v1 = min(t1, v0 + per);
  const uint16_t* zr = a.z + (size_t)r * a.ldz_r + (size_t)a.d * a.ldz_d;
  // the lane's range in batches of kRB entries, all loads of a batch issued first
  // (clamped to the range, masked after)
  constexpr int kRB = 16;
  double ms = 0.0;
  for (int vb = v0; vb < v1; vb += kRB) {
    uint16_t x[kRB];
#pragma unroll
    for (int j = 0; j < kRB; ++j) x[j] = zr[min(vb + j, v1 - 1)];
#pragma unroll
    for (int j = 0; j < kRB; ++j)
      if (vb + j < v1) ms += (double)fast_exp2(__builtin_fmaf(bf16_val(x[j]), a.cz, -H));
  }
  const double mi = wave_scan_incl(ms);
  const double me = mi - ms;
  const uint64_t hit2 = __ballot(ms > 0.0 && me <= tin && tin < mi);
  int tok = -1;
  if (hit2) {
    const int l = __ffsll((unsigned long long)hit2) - 1;
    if (lane == l) {
      double acc = me;
      for (int vb = v0; vb < v1 && tok < 0; vb += kRB) {
        uint16_t x[kRB];
#pragma unroll
        for (int j = 0; j < kRB; ++j) x[j] = zr[min(vb + j, v1 - 1)];
#pragma unroll
        for (int j = 0; j < kRB; ++j) {
          if (vb + j < v1 && tok < 0) {
            const double wv = (double)fast_exp2(__builtin_fmaf(bf16_val(x[j]), a.cz, -H));
            if (wv > 0.0 && tin < acc + wv) tok = vb + j;
            acc += wv;
          }
        }
      }
      if (tok < 0)  // rounding inside the lane: its last token with mass
        for (int v = v1 - 1; v >= v0 && tok < 0; --v)
          if (fast_exp2(__builtin_fmaf(bf16_val(zr[v]), a.cz, -H)) > 0.f) tok = v;
    }
    tok = __shfl(tok, l, 64);
  }
  if (tok < 0) {
    const uint64_t any = __ballot(ms > 0.0);
    if (any) {
      const int l = 63 - __clzll((long long)any);
      if (lane == l)
        for (int v = v1 - 1; v >= v0 && tok < 0; --v)
          if (fast_exp2(__builtin_fmaf(bf16_val(zr[v]), a.cz, -H)) > 0.f) tok = v;
      tok = __shfl(tok, l, 64);
    }
  }
  if (lane == 0) {
    *yo = tok;
    if (a.logq) {
      const double lse2 = (double)H + log2(total);
      const float lq = tok < 0 ? NAN : (float)(((double)bf16_val(zr[tok]) * (double)a.cz - lse2) * kLn2d);
      a.logq[(size_t)r * a.ld_y + a.d] = lq;
    }
    if (tok < 0) atomicOr(a.status, DSP_STATUS_NONFINITE);
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
  // row bounds of the next depth (NULL: none): probe tokens [R][D][4] of the L rows,
  // bounds written to theta[R * fn]
  const int32_t* probe;
  float* theta;
  int32_t D;
};

// Four probe tokens per (request, L row): probe j is the arg-max of the row over the
// 256-token blocks b with b % 4 == j (lowest id on ties), or -1 if none is finite.
// Four distinct tokens, so the smallest of any row's values at them is a lower bound
// on that row's 4th-largest value. One workgroup per (request, row, j).
struct ProbeArgs {
  const uint16_t* L;
  int64_t ldL_r, ldL_d;
  int32_t V, D, d0;   // rows d0 .. D-1
  int32_t* probe;     // [R][D][4]
};
__global__ __launch_bounds__(256) void tree_probe_kernel(ProbeArgs a) {
  __shared__ float s_v[4];
  __shared__ int32_t s_i[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = blockIdx.x & 3;
  const int nrow = a.D - a.d0;
  const int i = (blockIdx.x >> 2) / nrow, d = a.d0 + (blockIdx.x >> 2) % nrow;
  const uint16_t* row = a.L + (size_t)i * a.ldL_r + (size_t)d * a.ldL_d;
  const bool al = ((uintptr_t)row & 15) == 0;
  const int nb = (a.V + 255) / 256;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  // 32 threads per block (8 tokens each), 8 blocks per pass; a thread's tokens increase
  for (int b = j + 4 * (tid >> 5); b < nb; b += 32) {
    const int v0 = b * 256 + 8 * (tid & 31);
    float x[8];
    if (al && v0 + 8 <= a.V) {
      const u32x4 w = *(const u32x4*)(row + v0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(w[e]);
        x[2 * e + 1] = bf16_hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = v0 + e < a.V ? bf16_val(row[v0 + e]) : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (x[e] > best) {
        best = x[e];
        bi = v0 + e;
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, best, bi)) {
      best = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    s_v[wave] = best;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(s_v[w], s_i[w], best, bi)) {
        best = s_v[w];
        bi = s_i[w];
      }
    a.probe[((size_t)i * a.D + d) * 4 + j] = best == -INFINITY ? -1 : bi;
  }
}

// One workgroup per request: merge the column-group partials of its parents (16
// lanes per parent), score every candidate child in fp64 (4 lanes per candidate,
// each a quarter of the rank, every load issued before any is used), keep the top-F
// by (s desc, parent slot, child rank).
__global__ __launch_bounds__(256) void tree_merge_kernel(TreeMergeArgs a) {
  __shared__ double c_score[256];
  __shared__ int32_t c_tok[256];
  __shared__ double p_lse[64];
  __shared__ int32_t p_top[64][kTopK];
  __shared__ int32_t s_ntok[64];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int nc = a.fp * a.topk;
  const int qn = a.rank / 4;  // a multiple of 8
  // With one batch of candidates and of their rank quarters (nc <= 64, rank <= 256), the
  // parents' U rows that the candidates' dot products read are known from the start:
  // their loads are issued here, ahead of the partials, instead of after the merge.
  const bool upre_on = nc <= 64 && qn / 8 <= 8;
  u32x4 upre[8];
  if (upre_on) {
    const int c = tid >> 2, r = tid & 3;
    const int ptoken = a.ptok[i * a.fp + (c < nc ? c / a.topk : 0)];
    const u32x4* ur = (const u32x4*)(a.U + (size_t)ptoken * a.rank + r * qn);
#pragma unroll
    for (int t2 = 0; t2 < 8; ++t2) upre[t2] = ur[min(t2, qn / 8 - 1)];
  }
  // parents: 16 lanes each (aligned groups inside a wavefront), 16 parents per pass
  for (int pb = 0; pb < a.fp; pb += 16) {
    const int p = pb + (tid >> 4), j = tid & 15;
    const bool pv = p < a.fp;
    const TreePart* pr = a.part + (size_t)(i * a.fp + (pv ? p : 0)) * a.G;
    float tv[kTopK];
    int ti[kTopK];
#pragma unroll
    for (int q = 0; q < kTopK; ++q) {
      tv[q] = -INFINITY;
      ti[q] = 0x7fffffff;
    }
    float H = -INFINITY;
    float rf1[4];  // the first batch's (reference, sum) pairs, reused below when G <= 64
    double sm1[4];
    // four partials per lane per batch, loaded unconditionally (clamped, masked after:
    // a load under a branch is waited for on the spot)
    for (int g0 = j; g0 < a.G; g0 += 64) {
      TreePart tp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) tp[q] = pr[min(g0 + 16 * q, a.G - 1)];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (pv && g0 + 16 * q < a.G) {
          merge_top4(tv, ti, tp[q].val, tp[q].idx);
          H = fmaxf(H, tp[q].ref);
        }
        if (g0 == j) {
          rf1[q] = tp[q].ref;
          sm1[q] = tp[q].sum;
        }
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      float ov[kTopK];
      int oi[kTopK];
#pragma unroll
      for (int q = 0; q < kTopK; ++q) {
        ov[q] = __shfl_xor(tv[q], o, 64);
        oi[q] = __shfl_xor(ti[q], o, 64);
      }
      merge_top4(tv, ti, ov, oi);
      H = fmaxf(H, __shfl_xor(H, o, 64));
    }
    double S = 0.0;
    if (a.G <= 64) {  // one batch: the pairs are still in registers (same terms, same order)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (pv && j + 16 * q < a.G && rf1[q] != -INFINITY) S += sm1[q] * exp2((double)rf1[q] - (double)H);
    }
    for (int g0 = j; a.G > 64 && g0 < a.G; g0 += 64) {
      float rf[4];
      double sm[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = min(g0 + 16 * q, a.G - 1);
        rf[q] = pr[g].ref;
        sm[q] = pr[g].sum;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (pv && g0 + 16 * q < a.G && rf[q] != -INFINITY) S += sm[q] * exp2((double)rf[q] - (double)H);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) S += __shfl_xor(S, o, 64);
    if (pv && j == 0) {
      // a +inf or NaN in the row makes the maximum infinite or the sum NaN (the maxima
      // skip NaN, the exponentials do not): a fault; the children are then unspecified
      if (H == INFINITY || !(S == S) || S == INFINITY) atomicOr(a.status, DSP_STATUS_NONFINITE);
      p_lse[p] = ((double)H + log2(S)) * kLn2d;
#pragma unroll
      for (int q = 0; q < kTopK; ++q)  // below -2^127: a masked entry (staged as -max)
        p_top[p][q] = tv[q] < -0x1p127f ? -1 : ti[q];
    }
  }
  __syncthreads();
  // candidates: 4 lanes each, lane quarter r covers rank [r*rank/4, (r+1)*rank/4)
  for (int cb = 0; cb < nc; cb += 64) {
    const int c = cb + (tid >> 2), r = tid & 3;
    const bool cv = c < nc;
    const int p = cv ? c / a.topk : 0, rk = cv ? c % a.topk : 0;
    int v = p_top[p][rk];
    if (cv && (v < 0 || v >= a.V)) {  // fewer than topk finite entries, or non-finite scores
      if (r == 0) atomicOr(a.status, DSP_STATUS_NONFINITE);
    }
    if (v < 0 || v >= a.V) v = 0;
    const int ptoken = a.ptok[i * a.fp + p];
    const u32x4* ur = (const u32x4*)(a.U + (size_t)ptoken * a.rank + r * qn);
    const u32x4* wr = (const u32x4*)(a.Wt + (size_t)v * a.rank + r * qn);
    double m = 0.0;
    for (int j0 = 0; j0 < qn / 8; j0 += 8) {  // 8 vector pairs in flight (clamped, masked after)
      u32x4 uu[8], ww[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int tt = min(j0 + t, qn / 8 - 1);
        uu[t] = upre_on ? upre[t] : ur[tt];  // the same vectors (one batch: j0 = 0)
        ww[t] = wr[tt];
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (j0 + t < qn / 8)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            m += (double)bf16_lo(uu[t][h]) * (double)bf16_lo(ww[t][h]);
            m += (double)bf16_hi(uu[t][h]) * (double)bf16_hi(ww[t][h]);
          }
    }
    m += __shfl_xor(m, 1, 64);
    m += __shfl_xor(m, 2, 64);
    if (cv && r == 0) {
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
      s_ntok[rank] = c_tok[tid];
      a.ntok[i * a.fn + rank] = c_tok[tid];
      a.nscore[i * a.fn + rank] = s;
      Kept k;
      k.token = c_tok[tid];
      k.parent = a.d == 1 ? -1 : (a.d - 2) * a.F + p;
      k.score = s;
      a.kept[(size_t)i * a.kept_stride + (size_t)(a.d - 1) * a.F + rank] = k;
    }
  }
  if (!a.theta) return;
  __syncthreads();
  // Row bounds for the next depth (L row a.d): for new parent r and probe j, z = L + U[tok]
  // . W exactly (fp64, 4 lanes per pair), less 2^-12 (|L| + sum |u w|), which exceeds
  // the error of any fp32 evaluation of the 257-term sum; the bound of r is the smallest
  // over its four probes, rounded down to fp32 and stepped below (entries >= it pass).
  const int32_t* pr = a.probe + ((size_t)i * a.D + a.d) * 4;
  for (int pb = 0; pb < a.fn * 4; pb += 64) {
    const int pj = pb + (tid >> 2), qr = tid & 3;
    const bool ok = pj < a.fn * 4;
    const int r = ok ? pj >> 2 : 0;
    const int v = ok ? pr[pj & 3] : -1;
    double m = 0.0, am = 0.0;
    {
      // loads unconditional (token 0 stands in for a missing probe, masked after)
      const int qn = a.rank / 4;
      const u32x4* ur = (const u32x4*)(a.U + (size_t)s_ntok[r] * a.rank + qr * qn);
      const u32x4* wr = (const u32x4*)(a.Wt + (size_t)(v >= 0 ? v : 0) * a.rank + qr * qn);
      for (int j0 = 0; j0 < qn / 8; j0 += 8) {
        u32x4 uu[8], ww[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int tt = min(j0 + t, qn / 8 - 1);
          uu[t] = ur[tt];
          ww[t] = wr[tt];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (j0 + t < qn / 8)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const double p0 = (double)bf16_lo(uu[t][h]) * (double)bf16_lo(ww[t][h]);
              const double p1 = (double)bf16_hi(uu[t][h]) * (double)bf16_hi(ww[t][h]);
              m += p0 + p1;
              am += fabs(p0) + fabs(p1);
            }
      }
    }
    m += __shfl_xor(m, 1, 64);
    m += __shfl_xor(m, 2, 64);
    am += __shfl_xor(am, 1, 64);
    am += __shfl_xor(am, 2, 64);
    double bound = -INFINITY;
    if (v >= 0) {
      const double l = (double)bf16_val(a.L[(size_t)i * a.ldL_r + (size_t)a.d * a.ldL_d + v]);
      bound = l + m - 0x1p-12 * (fabs(l) + am);
    }
    bound = fmin(bound, __shfl_xor(bound, 4, 64));
    bound = fmin(bound, __shfl_xor(bound, 8, 64));
    if (ok && (tid & 15) == 0) {
      float t = (float)bound;
      if ((double)t > bound) t = nextafterf(t, -INFINITY);
      a.theta[i * a.fn + r] = nextafterf(t, -INFINITY);
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
  uint64_t* anc_mask;  // nullable: [R, topN, W] ancestor-or-self bit sets, W = ceil(topN / 64)
};

__global__ __launch_bounds__(256) void tree_final_kernel(TreeFinalArgs a) {
  __shared__ double s_score[1024];
  __shared__ int32_t s_valid[1024];
  __shared__ int32_t s_out[1024];
  __shared__ int32_t fsz[1024];
  __shared__ int32_t s_par[1024];  // parent of each output node, in output order
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
  // rank by (score desc, depth asc, slot asc) == (score desc, kept id asc). Each
  // depth's frontier is already in that order (slot = rank of the pruning), so the
  // rank of a node is its slot plus, for every other depth, a binary-search count of
  // the nodes there that precede it: score >= s at shallower depths (they win ties),
  // score > s at deeper ones.
  for (int e = tid; e < nk; e += 256) {
    if (!s_valid[e]) continue;
    const double s = s_score[e];
    const int de = e / a.F;
    int rank = e % a.F;
    for (int d = 0; d < a.D; ++d) {
      if (d == de) continue;
      const double* ls = s_score + d * a.F;
      int lo = 0, hi = fsz[d];  // first slot that does not precede e
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const bool pre = d < de ? ls[mid] >= s : ls[mid] > s;
        if (pre) lo = mid + 1;
        else hi = mid;
      }
      rank += lo;
    }
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
    const int po = k.parent < 0 ? -1 : s_out[k.parent];
    a.node_token[at] = k.token;
    a.node_parent[at] = po;
    a.node_depth[at] = e / a.F + 1;
    a.node_score[at] = k.score;
    s_par[o] = po;
  }
  for (int o = nout + tid; o < a.topN; o += 256) {
    const size_t at = (size_t)i * a.topN + o;
    a.node_token[at] = -1;
    a.node_parent[at] = -1;
    a.node_depth[at] = 0;
    a.node_score[at] = 0.0;
  }
  if (tid == 0) a.n_nodes[i] = nout;
  if (a.anc_mask) {
    // node o sees itself and its ancestors (tree-causal attention in the verify's
    // target forward): per word, walk the parent chain (parent[o] < o) and collect the
    // bits that fall in that word
    __syncthreads();
    const int W = (a.topN + 63) / 64;
    for (int o = tid; o < a.topN; o += 256) {
      uint64_t* mo = a.anc_mask + ((size_t)i * a.topN + o) * W;
      for (int w = 0; w < W; ++w) {
        uint64_t m = 0;
        if (o < nout)
          for (int c = o; c >= 0 && c >= 64 * w; c = s_par[c])
            if (c < 64 * (w + 1)) m |= 1ull << (c & 63);
        mo[w] = m;
      }
    }
  }
}

// k-steps of 16 for a rank (rank padded with zeros to a power of two >= 32)
int ksteps(int rank) {
  int ks = 2;
  while (16 * ks < rank) ks *= 2;
  return ks;
}

// ---------------------------------------------------------------- RNN head
// The memo update of the RNN sequential head (DSpark study notes, section 4):
//   s_d = tanh(s_{d-1} A + E[y_{d-1}] + h_d G + b),  s_0 = 0,
// in fp64 throughout (bf16 inputs widen exactly), so the memo agrees with any other
// fp64 evaluation to rounding of the last bits; it enters the vocabulary projection
// rounded to bf16 (nearest, ties to even), through the Markov GEMM with the memo rows
// as the parent rows' factor rows.

// P[m, j] = sum_k h[m, k] Gt[j, k] for m = (request, position) rows: a fp64 GEMM tile of
// 64 rows x 64 memo entries per 256-thread workgroup, 4 x 4 outputs per thread. k moves
// in chunks of 64: each thread fetches its two 16-byte vectors of h and of Gt for the
// next chunk while the current one (widened to fp32 in LDS, exact for bf16) is used.
struct RnnProjArgs {
  const uint16_t* h;
  int64_t ldh_r, ldh_k;
  int32_t H, n;            // hidden size, positions per request
  const uint16_t* Gt;      // [r, H]
  int32_t rank, rows;      // rows = R * n
  double* P;               // [rows, rank]
};
constexpr int kPT = 64;    // tile rows / columns
constexpr int kPK = 64;    // k per chunk

__global__ __launch_bounds__(256) void rnn_proj_kernel(RnnProjArgs a) {
  __shared__ float sh[kPK][kPT + 4];
  __shared__ float sg[kPK][kPT + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.x * kPT, j0 = blockIdx.y * kPT;
  // this thread's two (row, 8-k group) slots of each tile: slot e = tid + 256 q covers
  // row e / 8 and k = 8 (e % 8) .. + 8
  const bool vec = (a.H % 8) == 0 && (a.ldh_k % 8) == 0 && (a.ldh_r % 8) == 0 &&
                   ((uintptr_t)a.h % 16) == 0 && ((uintptr_t)a.Gt % 16) == 0;
  auto fetch = [&](int k0, uint32_t (*hv)[4], uint32_t (*gv)[4]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q, rr = e >> 3, kk = 8 * (e & 7), k = k0 + kk;
      const int m = m0 + rr, j = j0 + rr;
      const int i = m / a.n, d = m % a.n;
      const uint16_t* hp = a.h + (size_t)i * a.ldh_r + (size_t)d * a.ldh_k + k;
      const uint16_t* gp = a.Gt + (size_t)j * a.H + k;
      if (vec && m < a.rows && k + 8 <= a.H) {
        const uint4 w = *(const uint4*)hp;
        hv[q][0] = w.x; hv[q][1] = w.y; hv[q][2] = w.z; hv[q][3] = w.w;
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t lo = (m < a.rows && k + 2 * t < a.H) ? hp[2 * t] : 0u;
          const uint32_t hi = (m < a.rows && k + 2 * t + 1 < a.H) ? hp[2 * t + 1] : 0u;
          hv[q][t] = lo | (hi << 16);
        }
      }
      if (vec && j < a.rank && k + 8 <= a.H) {
        const uint4 w = *(const uint4*)gp;
        gv[q][0] = w.x; gv[q][1] = w.y; gv[q][2] = w.z; gv[q][3] = w.w;
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t lo = (j < a.rank && k + 2 * t < a.H) ? gp[2 * t] : 0u;
          const uint32_t hi = (j < a.rank && k + 2 * t + 1 < a.H) ? gp[2 * t + 1] : 0u;
          gv[q][t] = lo | (hi << 16);
        }
      }
    }
  };
  double acc[4][4] = {};
  uint32_t hv[2][4], gv[2][4];
  fetch(0, hv, gv);
  for (int k0 = 0; k0 < a.H; k0 += kPK) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q, rr = e >> 3, kk = 8 * (e & 7);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sh[kk + 2 * t][rr] = bf16_lo(hv[q][t]);
        sh[kk + 2 * t + 1][rr] = bf16_hi(hv[q][t]);
        sg[kk + 2 * t][rr] = bf16_lo(gv[q][t]);
        sg[kk + 2 * t + 1][rr] = bf16_hi(gv[q][t]);
      }
    }
    __syncthreads();
    if (k0 + kPK < a.H) fetch(k0 + kPK, hv, gv);  // in flight during this chunk's products
#pragma unroll 8
    for (int kk = 0; kk < kPK; ++kk) {
      const float4 h4 = *(const float4*)&sh[kk][ty * 4];
      const float4 g4 = *(const float4*)&sg[kk][tx * 4];
      const double hr[4] = {(double)h4.x, (double)h4.y, (double)h4.z, (double)h4.w};
      const double gc[4] = {(double)g4.x, (double)g4.y, (double)g4.z, (double)g4.w};
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = __builtin_fma(hr[p], gc[q], acc[p][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + ty * 4 + p, j = j0 + tx * 4 + q;
      if (m < a.rows && j < a.rank) a.P[(size_t)m * a.rank + j] = acc[p][q];
    }
}

struct RnnMemoArgs {
  const int32_t* prev;     // previous token of each request at prev[i * ld_prev]
  int64_t ld_prev;
  const uint16_t* A;       // [r, r]
  const uint16_t* E;       // [V, r]
  const float* bias;       // [r] or NULL
  const double* P;         // [R * n, r]
  int32_t n, d, rank, V;
  double* memo;            // [R, r] fp64, updated in place
  uint16_t* memo_bf;       // [R, r] bf16 bits for the projection
  int32_t* idx;            // [R]: row i of the memo table for parent row i
  int32_t* status;
};

// fp64 -> bf16, nearest with ties to even, in one rounding: round to fp32 toward zero,
// make it odd if that was inexact (round to odd keeps the two extra bits the final
// rounding needs), then the usual fp32 -> bf16 nearest-even.
__device__ __forceinline__ uint16_t bf16_from_double(double x) {
  float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(256) void rnn_memo_kernel(RnnMemoArgs a) {
  extern __shared__ double sprev[];  // [rank]
  const int i = blockIdx.x, tid = threadIdx.x;
  double* mrow = a.memo + (size_t)i * a.rank;
  for (int k = tid; k < a.rank; k += 256) sprev[k] = a.d == 0 ? 0.0 : mrow[k];
  int tok = a.prev[(size_t)i * a.ld_prev];
  if (tok < 0 || tok >= a.V) {
    if (tid == 0) atomicOr(a.status, DSP_STATUS_TOKEN_RANGE);
    tok = 0;
  }
  if (tid == 0) a.idx[i] = i;
  __syncthreads();
  const double* prow = a.P + ((size_t)i * a.n + a.d) * a.rank;
  for (int j = tid; j < a.rank; j += 256) {
    double pre = 0.0;
    // 32 loads of A in flight, then their products in order (rank is a multiple of 32)
    for (int k0 = 0; k0 < a.rank; k0 += 32) {
      uint16_t av[32];
#pragma unroll
      for (int q = 0; q < 32; ++q) av[q] = a.A[(size_t)(k0 + q) * a.rank + j];
#pragma unroll
      for (int q = 0; q < 32; ++q) pre = __builtin_fma(sprev[k0 + q], (double)bf16_val(av[q]), pre);
    }
    pre += (double)bf16_val(a.E[(size_t)tok * a.rank + j]);
    pre += prow[j];
    if (a.bias) pre += (double)a.bias[j];
    const double sj = tanh(pre);
    mrow[j] = sj;
    a.memo_bf[(size_t)i * a.rank + j] = bf16_from_double(sj);
  }
}

size_t gemm_lds_bytes(int ks, int mode) {
  return (size_t)2 * (kTS * 2 * ks + kTR * 4) * 16 + (mode == MODE_SAMPLE ? (size_t)kWaves * 32 * kZS : 0);
}

int pick_groups(int rows, int V) {
  const int nrb = (rows + kTR - 1) / kTR;
  const int nst = (V + kTS - 1) / kTS;
  int G = (kTargetWGs + nrb - 1) / nrb;
  if (nrb > 1 && G >= 8) G = G / 8 * 8;
  if (G > nst) G = nst;
  if (G < 1) G = 1;
  return G;
}

template <int MODE, int KS, bool LAL, bool LTM = false>
int32_t launch_gemm_ks(int kid, GemmArgs a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)markov_gemm_kernel<MODE, KS, LAL, LTM>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  a.nrb = (a.rows + kTR - 1) / kTR;
  a.xcd_map = a.nrb > 1 && a.G % 8 == 0;
  launch(kid, markov_gemm_kernel<MODE, KS, LAL, LTM>, dim3((unsigned)(a.G * a.nrb)), dim3(kGT),
         (uint32_t)gemm_lds_bytes(KS, MODE), s, a);
  return hip_check(hipGetLastError(), "markov gemm launch");
}

template <int MODE, bool LAL>
int32_t launch_gemm_al(int kid, const GemmArgs& a, hipStream_t s) {
  switch (ksteps(a.rank)) {
    case 2: return launch_gemm_ks<MODE, 2, LAL>(kid, a, s);
    case 4: return launch_gemm_ks<MODE, 4, LAL>(kid, a, s);
    case 8: return launch_gemm_ks<MODE, 8, LAL>(kid, a, s);
    case 16: return launch_gemm_ks<MODE, 16, LAL>(kid, a, s);
    default: return launch_gemm_ks<MODE, 32, LAL>(kid, a, s);
  }
}

// Every row block of kTR parent rows spans at most 16 requests (tree_gemm_kernel's L tile).
bool blocks_span_16(const GemmArgs& a) {
  for (int r0 = 0; r0 < a.rows; r0 += kTR) {
    const int rlast = (r0 + kTR < a.rows ? r0 + kTR : a.rows) - 1;
    if (rlast / a.rows_per_req - r0 / a.rows_per_req >= 16) return false;
  }
  return true;
}

size_t tree_split_lds_bytes(int ks) {
  const int wslot = kTS * 2 * ks > kGT ? kTS * 2 * ks : kGT;
  return ((size_t)6 * wslot + 6 * 64) * 16;  // six stage slots: Wt and the 1 KB L tile
}

template <int KS>
int32_t launch_tree_split_ks(int kid, GemmArgs a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)tree_gemm_kernel<KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    attr_set = true;
  }
  a.nrb = (a.rows + kTR - 1) / kTR;
  a.xcd_map = a.nrb > 1 && a.G % 8 == 0;
  launch(kid, tree_gemm_kernel<KS>, dim3((unsigned)(a.G * a.nrb)), dim3(kGT), (uint32_t)tree_split_lds_bytes(KS), s,
         a);
  return hip_check(hipGetLastError(), "tree gemm launch");
}

int32_t launch_tree_split(int kid, const GemmArgs& a, hipStream_t s) {
  switch (ksteps(a.rank)) {
    case 2: return launch_tree_split_ks<2>(kid, a, s);
    case 4: return launch_tree_split_ks<4>(kid, a, s);
    case 8: return launch_tree_split_ks<8>(kid, a, s);
    default: return launch_tree_split_ks<16>(kid, a, s);
  }
}

size_t chain_sched_lds_bytes(int ks) {
  const int wslot = kTS * 2 * ks > kGT ? kTS * 2 * ks : kGT;
  return ((size_t)4 * wslot + 4 * kTR * 4) * 16;  // four stage slots: Wt and the 16 KB L tile
}

template <int KS>
int32_t launch_chain_sched_ks(int kid, GemmArgs a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)chain_gemm_kernel<KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    attr_set = true;
  }
  a.nrb = (a.rows + kTR - 1) / kTR;
  a.xcd_map = a.nrb > 1 && a.G % 8 == 0;
  launch(kid, chain_gemm_kernel<KS>, dim3((unsigned)(a.G * a.nrb)), dim3(kGT), (uint32_t)chain_sched_lds_bytes(KS), s,
         a);
  return hip_check(hipGetLastError(), "chain gemm launch");
}

int32_t launch_chain_sched(int kid, const GemmArgs& a, hipStream_t s) {
  switch (ksteps(a.rank)) {
    case 2: return launch_chain_sched_ks<2>(kid, a, s);
    case 4: return launch_chain_sched_ks<4>(kid, a, s);
    case 8: return launch_chain_sched_ks<8>(kid, a, s);
    default: return launch_chain_sched_ks<16>(kid, a, s);
  }
}

// L rows 16-byte aligned (base and both strides) take the vector-load kernel
template <int MODE>
int32_t launch_gemm(int kid, const GemmArgs& a, hipStream_t s) {
  if ((size_t)a.V * a.rank * 2 >= kOOB)
    return fail(DSP_ERR_SHAPE, "Wt must span less than 2 GiB (V * rank * 2 bytes)");
  // token-major base logits (checked by the entry point: rank 256, aligned, span)
  if (a.l_tm) return launch_gemm_ks<MODE, 16, true, true>(kid, a, s);
  const size_t reqs = (size_t)(kTR + a.rows_per_req - 1) / a.rows_per_req + 1;  // requests a row block touches
  if ((reqs * (size_t)a.ldL_r + (size_t)a.V) * 2 >= kOOB)
    return fail(DSP_ERR_SHAPE, "the L rows of %d parent rows must span less than 2 GiB", kTR);
  const bool al = ((uintptr_t)a.L) % 16 == 0 && a.ldL_r % 8 == 0 && a.ldL_d % 8 == 0;
  if (MODE == MODE_TREE && al && ksteps(a.rank) <= 16 && option(DSP_OPT_TREE_SPLIT) && blocks_span_16(a))
    return launch_tree_split(kid, a, s);
  if (MODE == MODE_ARGMAX && al && ksteps(a.rank) <= 16 && option(DSP_OPT_CHAIN_SCHED)) return launch_chain_sched(kid, a, s);
  return al ? launch_gemm_al<MODE, true>(kid, a, s) : launch_gemm_al<MODE, false>(kid, a, s);
}

// Layout of the chain's base logits: row-major (DSP_BF16: element (i, d, v) at
// L + i*ldL_r + d*ldL_d + v) or token-major (DSP_BF16_TOKEN_MAJOR: at L + i + d*ldL_d +
// v*ldL_r). Returns DSP_OK or an error; *tm says which.
int32_t check_l_layout(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d, int32_t V, int32_t R,
                       int32_t n, int32_t rank, int32_t* tm) {
  *tm = l_dtype == DSP_BF16_TOKEN_MAJOR;
  if (!*tm) {
    if (ldL_d < V || ldL_r < (int64_t)(n - 1) * ldL_d + V) return fail(DSP_ERR_SHAPE, "L strides too small");
    return DSP_OK;
  }
  if (rank != 256) return fail(DSP_ERR_UNSUPPORTED, "token-major L is supported at rank 256");
  if (R % 8) return fail(DSP_ERR_SHAPE, "token-major L needs R a multiple of 8 (got %d)", R);
  if (ldL_r < R || ldL_d < (int64_t)(V - 1) * ldL_r + R) return fail(DSP_ERR_SHAPE, "token-major L strides too small");
  if (((uintptr_t)L) % 16 || ldL_r % 8 || ldL_d % 8)
    return fail(DSP_ERR_ALIGN, "token-major L: 16-byte aligned base, strides multiples of 8 elements");
  // the stage loads address one depth's tokens (plus a stage past V) from 32-bit offsets
  if ((((size_t)V + kTS) * ldL_r + kTR) * 2 >= kOOB)
    return fail(DSP_ERR_SHAPE, "token-major L of one depth must span less than 2 GiB");
  return DSP_OK;
}

int32_t check_markov_common(const void* L, int32_t l_dtype, const void* U, const void* Wt, int32_t V,
                            int32_t rank) {
  if (l_dtype != DSP_BF16 && l_dtype != DSP_BF16_TOKEN_MAJOR) return fail(DSP_ERR_DTYPE, "L must be bf16");
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
  size_t off_part, off_tok0, off_tok1, off_sc0, off_sc1, off_kept, off_probe, off_theta, total;
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
  t.off_probe = off; off = align_up(off + (size_t)R * D * 4 * sizeof(int32_t), 256);
  t.off_theta = off; off = align_up(off + (size_t)R * F * sizeof(float), 256);
  t.total = off;
  return t;
}

// ---------------------------------------------------------------- persistent chain (host)
// Workgroups of the persistent chain on the current device (one per CU, as many as there
// are 32-token tiles at most), or 0 when the path does not apply: it needs every CU's
// workgroup resident at once and at most kPMaxTiles tiles per workgroup.
int persist_groups(int V) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0, fit = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = -1;
    (void)hipFuncSetAttribute((const void*)chain_persist_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kPLds);
    (void)hipFuncSetAttribute((const void*)chain_persist_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kPLds);
    if (n > 0 && hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, chain_persist_kernel<true>, kPThreads, kPLds) != hipSuccess)
      fit = 0;
    int fit2 = 0;
    if (n > 0 && hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit2, chain_persist_kernel<false>, kPThreads, kPLds) != hipSuccess)
      fit2 = 0;
    cus[dev] = n > 0 && fit >= 1 && fit2 >= 1 ? (n < kTargetWGs ? n : kTargetWGs) : -1;
  }
  if (cus[dev] < 0) return 0;
  const int nst = (V + 31) / 32;
  const int G = nst < cus[dev] ? nst : cus[dev];
  return (nst + G - 1) / G <= kPMaxTiles ? G : 0;
}

struct PersistLayout {
  size_t off_part, off_keys, off_bar, total;
};
PersistLayout persist_layout(int R, int n_steps) {
  PersistLayout l;
  size_t off = 0;
  l.off_part = off;
  off = align_up(off + (size_t)n_steps * R * kTargetWGs * sizeof(ChainPart), 256);
  l.off_keys = off;
  off = align_up(off + (size_t)n_steps * kPGroups * R * kPKeyStride * sizeof(uint64_t), 256);
  l.off_bar = off;
  off = align_up(off + sizeof(uint32_t), 256);
  l.total = off;
  return l;
}

// Shapes the persistent chain takes (the device-side checks are in persist_groups).
bool persist_shape_ok(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d, int32_t V, int32_t rank,
                      int32_t R, int32_t n_steps) {
  if (l_dtype != DSP_BF16 || rank != 256 || R > kPMaxR) return false;
  if (((uintptr_t)L) % 16 || ldL_r % 8 || ldL_d % 8) return false;
  return (((size_t)(R - 1) * ldL_r + (size_t)(n_steps - 1) * ldL_d + V) * 2) < kOOB;
}

int32_t chain_persistent(int G, const void* L, int64_t ldL_r, int64_t ldL_d, const void* U, const void* Wt,
                         int32_t V, const int32_t* prev_tok, int32_t R, int32_t n_steps, int32_t* y, int64_t ld_y,
                         float* logq, int32_t* status, void* ws, hipStream_t s) {
  const PersistLayout l = persist_layout(R, n_steps);
  char* base = (char*)ws;
  PersistInitArgs ia{(uint64_t*)(base + l.off_keys), (size_t)n_steps * kPGroups * R, (uint32_t*)(base + l.off_bar)};
  launch(DSP_K_MARKOV_MERGE, chain_persist_init_kernel, dim3((unsigned)((ia.n_keys + 255) / 256)), dim3(256), 0, s,
         ia);
  int32_t rc = hip_check(hipGetLastError(), "persistent chain init launch");
  if (rc) return rc;
  PersistArgs pa{(const uint16_t*)U, (const uint16_t*)Wt, (const uint16_t*)L, ldL_r, ldL_d, prev_tok, V, R,
                 n_steps, G, (ChainPart*)(base + l.off_part), ia.keys, ia.bar,
                 (uint32_t)option(DSP_OPT_SPIN_LIMIT), status};
  if (logq)
    launch(DSP_K_CHAIN_PERSIST, chain_persist_kernel<true>, dim3((unsigned)G), dim3(kPThreads), (uint32_t)kPLds, s, pa);
  else
    launch(DSP_K_CHAIN_PERSIST, chain_persist_kernel<false>, dim3((unsigned)G), dim3(kPThreads), (uint32_t)kPLds, s, pa);
  rc = hip_check(hipGetLastError(), "persistent chain launch");
  if (rc) return rc;
  if (logq) {  // y and log q from the workgroups' partials
    ChainMergeArgs ma{pa.part, G, R, 0, y, ld_y, logq};
    launch(DSP_K_MARKOV_MERGE, chain_merge_kernel, dim3((unsigned)R, (unsigned)n_steps), dim3(64), 0, s, ma);
  } else {    // y from the keys
    PersistYArgs ya{ia.keys, R, n_steps, y, ld_y};
    launch(DSP_K_MARKOV_MERGE, chain_persist_y_kernel, dim3((unsigned)((R * n_steps + 255) / 256)), dim3(256), 0,
           s, ya);
  }
  return hip_check(hipGetLastError(), "chain merge launch");
}

}  // namespace
}  // namespace dsp

using namespace dsp;

extern "C" size_t dsp_draft_markov_step_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps,
                                                       int32_t want_logq) {
  (void)want_logq;
  if (R < 1 || V < 1) return 0;
  size_t need = align_up((size_t)pick_groups(R, V) * R * sizeof(ChainPart), 256);
  if (rank == 256 && R <= kPMaxR && n_steps >= 1) {
    const size_t p = persist_layout(R, n_steps).total;
    need = p > need ? p : need;
  }
  return need;
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
  int32_t tm = 0;
  rc = check_l_layout(L, l_dtype, ldL_r, ldL_d, V, R, n_steps, rank, &tm);
  if (rc) return rc;
  const size_t need = dsp_draft_markov_step_workspace_size(R, V, rank, n_steps, logq != nullptr);
  if (!ws || ws_bytes < need) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  hipStream_t s = (hipStream_t)stream;
  if (option(DSP_OPT_CHAIN_PERSISTENT) && persist_shape_ok(L, l_dtype, ldL_r, ldL_d, V, rank, R, n_steps)) {
    const int Gp = persist_groups(V);
    if (Gp > 0)
      return chain_persistent(Gp, L, ldL_r, ldL_d, U, Wt, V, prev_tok, R, n_steps, y, ld_y, logq, status, ws, s);
  }
  const int G = pick_groups(R, V);
  for (int d = 0; d < n_steps; ++d) {
    GemmArgs ga{(const uint16_t*)U, (const uint16_t*)Wt, V, rank,
                d == 0 ? prev_tok : y + (d - 1), d == 0 ? 1 : ld_y,
                (const uint16_t*)L, ldL_r, ldL_d, d, R, 1, G, ws, status};
    ga.l_tm = tm;
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

struct RnnLayout {
  size_t off_part, off_P, off_memo, off_bf, off_idx, total;
};
static RnnLayout rnn_layout(int R, int V, int rank, int n) {
  RnnLayout L;
  size_t off = 0;
  L.off_part = off;
  off = align_up(off + (size_t)pick_groups(R, V) * R * sizeof(ChainPart), 256);
  L.off_P = off;
  off = align_up(off + (size_t)R * n * rank * sizeof(double), 256);
  L.off_memo = off;
  off = align_up(off + (size_t)R * rank * sizeof(double), 256);
  L.off_bf = off;
  off = align_up(off + (size_t)R * rank * sizeof(uint16_t), 256);
  L.off_idx = off;
  off = align_up(off + (size_t)R * sizeof(int32_t), 256);
  L.total = off;
  return L;
}

extern "C" size_t dsp_draft_rnn_step_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps) {
  if (R < 1 || V < 1 || rank < 1 || n_steps < 1) return 0;
  return rnn_layout(R, V, rank, n_steps).total;
}

extern "C" int32_t dsp_draft_rnn_step(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                                      const void* h, int32_t h_dtype, int64_t ldh_r, int64_t ldh_k, int32_t H,
                                      const void* Gt, const void* A, const void* E, const float* bias,
                                      const void* Wot, int32_t V, int32_t rank, const int32_t* prev_tok,
                                      int32_t R, int32_t n_steps, int32_t* y, int64_t ld_y, float* logq,
                                      int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int32_t rc = check_markov_common(L, l_dtype, E, Wot, V, rank);
  if (rc) return rc;
  if (h_dtype != DSP_BF16) return fail(DSP_ERR_DTYPE, "h must be bf16");
  if (!h || !Gt || !A) return fail(DSP_ERR_NULL, "h, Gt and A are required");
  if (H < 1) return fail(DSP_ERR_SHAPE, "H must be >= 1");
  if (R < 1 || n_steps < 1) return fail(DSP_ERR_SHAPE, "need R >= 1 and n_steps >= 1");
  if (!prev_tok || !y || !status) return fail(DSP_ERR_NULL, "prev_tok, y and status are required");
  if (ld_y < n_steps) return fail(DSP_ERR_SHAPE, "ld_y < n_steps");
  int32_t tm = 0;
  rc = check_l_layout(L, l_dtype, ldL_r, ldL_d, V, R, n_steps, rank, &tm);
  if (rc) return rc;
  if (ldh_k < H || ldh_r < (int64_t)(n_steps - 1) * ldh_k + H) return fail(DSP_ERR_SHAPE, "h strides too small");
  if (((uintptr_t)h) % 2 || ((uintptr_t)Gt) % 2 || ((uintptr_t)A) % 2) return fail(DSP_ERR_ALIGN, "h, Gt, A: 2-byte aligned");
  const RnnLayout lay = rnn_layout(R, V, rank, n_steps);
  if (!ws || ws_bytes < lay.total) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", lay.total);
  hipStream_t s = (hipStream_t)stream;
  ChainPart* part = (ChainPart*)((uintptr_t)ws + lay.off_part);
  double* P = (double*)((uintptr_t)ws + lay.off_P);
  double* memo = (double*)((uintptr_t)ws + lay.off_memo);
  uint16_t* mbf = (uint16_t*)((uintptr_t)ws + lay.off_bf);
  int32_t* idx = (int32_t*)((uintptr_t)ws + lay.off_idx);
  // the backbone states' contribution to every position's update, up front
  RnnProjArgs pa{(const uint16_t*)h, ldh_r, ldh_k, H, n_steps, (const uint16_t*)Gt, rank, R * n_steps, P};
  launch(DSP_K_RNN_PROJ, rnn_proj_kernel, dim3((unsigned)((R * n_steps + kPT - 1) / kPT), (unsigned)((rank + kPT - 1) / kPT)),
         dim3(256), 0, s, pa);
  rc = hip_check(hipGetLastError(), "rnn projection launch");
  if (rc) return rc;
  const int G = pick_groups(R, V);
  for (int d = 0; d < n_steps; ++d) {
    RnnMemoArgs ma{d == 0 ? prev_tok : y + (d - 1), d == 0 ? 1 : ld_y, (const uint16_t*)A, (const uint16_t*)E,
                   bias, P, n_steps, d, rank, V, memo, mbf, idx, status};
    launch(DSP_K_RNN_MEMO, rnn_memo_kernel, dim3(R), dim3(256), (uint32_t)(rank * sizeof(double)), s, ma);
    rc = hip_check(hipGetLastError(), "rnn memo launch");
    if (rc) return rc;
    GemmArgs ga{mbf, (const uint16_t*)Wot, V, rank, idx, 1, (const uint16_t*)L, ldL_r, ldL_d, d, R, 1, G, part,
                status};
    ga.u_rows = R;
    ga.l_tm = tm;
    rc = logq ? launch_gemm<MODE_ARGMAX_LSE>(DSP_K_MARKOV_GEMM, ga, s)
              : launch_gemm<MODE_ARGMAX>(DSP_K_MARKOV_GEMM, ga, s);
    if (rc) return rc;
    ChainMergeArgs mg{part, G, R, d, y, ld_y, logq};
    launch(DSP_K_MARKOV_MERGE, chain_merge_kernel, dim3(R), dim3(64), 0, s, mg);
    rc = hip_check(hipGetLastError(), "chain merge launch");
    if (rc) return rc;
  }
  return DSP_OK;
}

extern "C" size_t dsp_draft_markov_sample_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps) {
  (void)rank;
  (void)n_steps;
  if (R < 1 || V < 1) return 0;
  return align_up((size_t)pick_groups(R, V) * R * sizeof(ChainPart), 256);
}

extern "C" int32_t dsp_draft_markov_sample(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                                           const void* U, const void* Wt, int32_t V, int32_t rank,
                                           const int32_t* prev_tok, int32_t R, int32_t n_steps,
                                           float temperature, uint64_t seed, uint64_t round,
                                           const uint64_t* round_dev, const int64_t* req_id, int32_t* y,
                                           int64_t ld_y, float* logq, void* z, int64_t ldz_r, int64_t ldz_d,
                                           int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int32_t rc = check_markov_common(L, l_dtype, U, Wt, V, rank);
  if (rc) return rc;
  if (R < 1 || n_steps < 1) return fail(DSP_ERR_SHAPE, "need R >= 1 and n_steps >= 1");
  if (!(temperature > 0.f) || temperature == INFINITY)
    return fail(DSP_ERR_SHAPE, "temperature must be finite and > 0 (use the greedy chain for T = 0)");
  if (!prev_tok || !y || !z || !status) return fail(DSP_ERR_NULL, "prev_tok, y, z and status are required");
  if (ld_y < n_steps) return fail(DSP_ERR_SHAPE, "ld_y < n_steps");
  int32_t tm = 0;
  rc = check_l_layout(L, l_dtype, ldL_r, ldL_d, V, R, n_steps, rank, &tm);
  if (rc) return rc;
  if (ldz_d < V || ldz_r < (int64_t)(n_steps - 1) * ldz_d + V) return fail(DSP_ERR_SHAPE, "z strides too small");
  if (((uintptr_t)z) % 16 || ldz_d % 8 || ldz_r % 8)
    return fail(DSP_ERR_ALIGN, "z must be 16-byte aligned with strides that are multiples of 8 elements");
  const size_t need = dsp_draft_markov_sample_workspace_size(R, V, rank, n_steps);
  if (!ws || ws_bytes < need) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  hipStream_t s = (hipStream_t)stream;
  const int G = pick_groups(R, V);
  const float cz = (float)(1.4426950408889634074 / (double)temperature);
  for (int d = 0; d < n_steps; ++d) {
    GemmArgs ga{(const uint16_t*)U, (const uint16_t*)Wt, V, rank,
                d == 0 ? prev_tok : y + (d - 1), d == 0 ? 1 : ld_y,
                (const uint16_t*)L, ldL_r, ldL_d, d, R, 1, G, ws, status};
    ga.l_tm = tm;
    ga.zout = (uint16_t*)z;
    ga.ldz_r = ldz_r;
    ga.ldz_d = ldz_d;
    ga.cz = cz;
    rc = launch_gemm<MODE_SAMPLE>(DSP_K_MARKOV_GEMM, ga, s);
    if (rc) return rc;
    ChainSampleArgs sa{(const ChainPart*)ws, G, R, d, V, (const uint16_t*)z, ldz_r, ldz_d, cz,
                       seed, round, round_dev, req_id, y, ld_y, logq, status};
    launch(DSP_K_MARKOV_MERGE, chain_sample_kernel, dim3(R), dim3(64), 0, s, sa);
    rc = hip_check(hipGetLastError(), "chain sample launch");
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
                                   int32_t* n_nodes, uint64_t* anc_mask, int32_t* status, void* ws,
                                   size_t ws_bytes, void* stream) {
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
  if (l_dtype != DSP_BF16) return fail(DSP_ERR_UNSUPPORTED, "the tree takes row-major L");
  if (ldL_d < V || ldL_r < (int64_t)(D - 1) * ldL_d + V) return fail(DSP_ERR_SHAPE, "L strides too small");
  const TreeLayout T = tree_layout(R, D, V, rank, topk, frontier);
  if (!ws || ws_bytes < T.total) return fail(DSP_ERR_WORKSPACE, "workspace needs %zu bytes", T.total);
  hipStream_t s = (hipStream_t)stream;
  const uintptr_t b = (uintptr_t)ws;
  TreePart* part = (TreePart*)(b + T.off_part);
  int32_t* tok[2] = {(int32_t*)(b + T.off_tok0), (int32_t*)(b + T.off_tok1)};
  double* sc[2] = {(double*)(b + T.off_sc0), (double*)(b + T.off_sc1)};
  Kept* kept = (Kept*)(b + T.off_kept);
  int32_t* probe = (int32_t*)(b + T.off_probe);
  float* theta = (float*)(b + T.off_theta);
  int f[1024];
  frontier_sizes(D, topk, frontier, f);
  // probe tokens of the L rows of depths 2..D (row bounds for the top-4 selection)
  if (D > 1) {
    ProbeArgs pa{(const uint16_t*)L, ldL_r, ldL_d, V, D, 1, probe};
    if ((int64_t)R * (D - 1) * 4 >= (int64_t)1 << 31) return fail(DSP_ERR_SHAPE, "R * D too large");
    launch(DSP_K_TREE_PROBE, tree_probe_kernel, dim3((unsigned)(R * (D - 1) * 4)), dim3(256), 0, s, pa);
    rc = hip_check(hipGetLastError(), "tree probe launch");
    if (rc) return rc;
  }
  int fp = 1;
  for (int d = 1; d <= D; ++d) {
    const int rows = R * fp;
    const int G = pick_groups(rows, V);
    const int32_t* ptok = d == 1 ? anchor : tok[d & 1];
    GemmArgs ga{(const uint16_t*)U, (const uint16_t*)Wt, V, rank, ptok, 1, (const uint16_t*)L, ldL_r,
                ldL_d, d - 1, rows, fp, G, part, status};
    ga.theta = d == 1 ? nullptr : theta;
    rc = launch_gemm<MODE_TREE>(DSP_K_TREE_GEMM, ga, s);
    if (rc) return rc;
    const int fn = f[d - 1];
    TreeMergeArgs ma{part, G, d, fp, fn, topk, frontier, R, V, rank, ptok, d == 1 ? nullptr : sc[d & 1],
                     tok[(d + 1) & 1], sc[(d + 1) & 1], kept, T.kept_stride, (const uint16_t*)L, ldL_r,
                     ldL_d, (const uint16_t*)U, (const uint16_t*)Wt, status, probe, d < D ? theta : nullptr, D};
    launch(DSP_K_TREE_MERGE, tree_merge_kernel, dim3(R), dim3(256), 0, s, ma);
    rc = hip_check(hipGetLastError(), "tree merge launch");
    if (rc) return rc;
    fp = fn;
  }
  TreeFinalArgs fa{kept, T.kept_stride, D, frontier, topk, topN, R, node_token, node_parent, node_depth,
                   node_score, n_nodes, anc_mask};
    launch(DSP_K_TREE_FINAL, tree_final_kernel, dim3(R), dim3(256), 0, s, fa);
  return hip_check(hipGetLastError(), "tree final launch");
}
