// Routing kernels: two-level top-k router and the stable per-bin token lists.
//
// Router ("Breaking the MoE LLM Trilemma", papernotes.org note, key design 3:
// groups first, then experts inside the chosen groups; FP32 router as in the
// MoE routing page "混合专家模型的路由机制与工程落地", section 3.1), in two
// kernels:
//   logits  every router score of every token, s = x . [W_grp | W_exp^0 ..
//           W_exp^{G-1}], as one MFMA GEMM with FP32 accuracy (fp32 MFMAs
//           for fp32 activations, split-bf16 MFMAs with FP32 accumulation
//           for 16-bit ones), k split over the wavefronts of a workgroup
//           and, for small batches, over workgroups;
//   select  the top groups of s_grp + c, then the top experts of each
//           chosen group's scores + b, larger score first, ties to the
//           lower index, NaN ranked last; gate weights are the product of
//           the two softmaxes over the chosen scores.  A wavefront per
//           token (butterfly top-k over the lanes) in the select kernel, a
//           thread per token where scores and selection share one kernel.
// Scoring the experts of every group (not only the chosen ones) costs
// G*K extra columns of a small fp32 GEMM and removes a dependent second
// pass over the weights.
//
// Token lists (dropless dispatch, tokens ascending within each bin): the
// select kernel counts assignments per (chunk of 256 assignments, bin) with
// atomics; the scatter kernel turns those counts into per-bin offsets with a
// prefix sum and places each assignment at offset + (assignments of the same
// bin in earlier chunks) + (its rank inside its own chunk), the rank coming
// from a wave ballot over equal bins, so the result does not depend on
// scheduling.
#include "common.h"
#include "kernels.h"

namespace cefn {

namespace {

// ------------------------------------------------------------- logits --
// Output blocks (32 score columns c, 32 tokens t) over depth k with
// v_mfma_f32_32x32x2f32: A[c][k] from the router matrix, B[k][t] from X.
// Sixteen k at a time: lane half h supplies k = base + 8h + s in step s, so
// a lane reads 8 consecutive activations of its token (16 bytes, once for
// every column block) and 8 consecutive (re-laid-out) weights of its column.
template <int XT>
__device__ __forceinline__ void load8x(const typename Elem<XT>::T* p, float (&v)[8]) {
  if constexpr (XT == DT_F32) {
    const f4v q0 = *reinterpret_cast<const f4v*>(p);
    const f4v q1 = *reinterpret_cast<const f4v*>(p + 4);
    v[0] = q0[0]; v[1] = q0[1]; v[2] = q0[2]; v[3] = q0[3];
    v[4] = q1[0]; v[5] = q1[1]; v[6] = q1[2]; v[7] = q1[3];
  } else {
    const u4v q = *reinterpret_cast<const u4v*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t b = static_cast<uint16_t>((q[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      v[e] = (XT == DT_F16) ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
    }
  }
}

// 16-bit activations: the same partial scores from bf16 MFMAs.  The FP32
// router matrix is held as three bf16 parts (W = p0 + p1 + p2 to within
// 2^-24 relative); bf16 activations enter as they are, fp16 ones as two
// exact bf16 parts (an fp16 significand has 11 bits: the nearest bf16 and
// the at most 4-bit remainder).  A product of two bf16 is exact in FP32,
// so the FP32 accumulation of x.p0 + x.p1 + x.p2 (+ xr.p0 + xr.p1 for fp16)
// differs from an FP32 dot product only by the order of the additions and
// by terms below 2^-24 of the score, as the FP32 router requires, at a
// fraction of the FP32 MFMA time.
// TBN consecutive token blocks (tb .. tb + TBN - 1) share each load of the
// router matrix parts: for large batches the parts, re-read once per token
// block, are most of the bytes a compute unit loads.  Each block's MFMA
// sequence is the same as with TBN = 1, so its scores are bit for bit the
// same.
template <int XT, int NCB, int TBN = 1>
__device__ __forceinline__ void score_tiles_bf(const RouteArgs& a, int tb, int cb0, int k0, int kq, int lane,
                                               f16v (&acc)[TBN][NCB]) {
  using XE = typename Elem<XT>::T;
  using B8 = typename Frag<DT_BF16>::T;
  const int h = lane >> 5;
  const XE* xp[TBN];
#pragma unroll
  for (int b = 0; b < TBN; ++b) {
    int tok = (tb + b) * 32 + (lane & 31);
    tok = tok < a.T ? tok : a.T - 1;  // rows past the batch repeat the last one
    xp[b] = static_cast<const XE*>(a.X) + (long)tok * a.d + k0 + 8 * h;
  }
  const long pstride = (long)(a.d / 16) * a.NCp * 16;
  const uint16_t* wp = a.Wb + ((long)(k0 / 16) * a.NCp + cb0 * 32 + (lane & 31)) * 16 + 8 * h;
  const long wstep = (long)a.NCp * 16;
#pragma unroll
  for (int b = 0; b < TBN; ++b)
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][c][v] = 0.f;
  const int n16 = kq / 16;
  if (n16 == 0) return;
  auto issue = [&](int i, u4v (&xv)[TBN], u4v (&wv)[NCB][3]) {
    const int ic = i < n16 ? i : n16 - 1;  // the last group re-reads itself
#pragma unroll
    for (int b = 0; b < TBN; ++b) xv[b] = *reinterpret_cast<const u4v*>(xp[b] + ic * 16);
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int p = 0; p < 3; ++p) wv[c][p] = *reinterpret_cast<const u4v*>(wp + p * pstride + ic * wstep + c * 32 * 16);
  };
  // Each accumulator takes x.p0, x.p1, x.p2 (then xr.p0, xr.p1) in that
  // order; the loops run the parts outermost so that consecutive MFMAs
  // update different accumulators (back-to-back MFMAs on one accumulator
  // wait for each other's results).
  auto mma = [&](const u4v (&xv)[TBN], const u4v (&wv)[NCB][3]) {
    B8 xh[TBN], xl[TBN];
#pragma unroll
    for (int b = 0; b < TBN; ++b) {
      if constexpr (XT == DT_BF16) {
        xh[b] = __builtin_bit_cast(B8, xv[b]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t pr = xv[b][e >> 1];
          const float f = f16_bits_to_f32(static_cast<uint16_t>((pr >> (16 * (e & 1))) & 0xFFFFu));
          const uint16_t hb = f32_to_bf16_bits(f);
          xh[b][e] = __builtin_bit_cast(__bf16, hb);
          xl[b][e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(f - bf16_bits_to_f32(hb)));
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int b = 0; b < TBN; ++b)
#pragma unroll
        for (int c = 0; c < NCB; ++c) acc[b][c] = mfma32<DT_BF16>(__builtin_bit_cast(B8, wv[c][p]), xh[b], acc[b][c]);
    if constexpr (XT != DT_BF16) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int b = 0; b < TBN; ++b)
#pragma unroll
          for (int c = 0; c < NCB; ++c) acc[b][c] = mfma32<DT_BF16>(__builtin_bit_cast(B8, wv[c][p]), xl[b], acc[b][c]);
    }
  };
  // loads run PD groups of 16 k ahead of the MFMAs (a ring of PD + 1
  // register sets): two for one token block, whose group has few MFMAs; one
  // for two blocks (twice the MFMAs per group, and two workgroups per
  // compute unit fit only then)
  constexpr int PD = TBN > 1 ? 1 : 2, R = PD + 1;
  u4v xr[R][TBN];
  u4v wr[R][NCB][3];
#pragma unroll
  for (int p = 0; p < PD; ++p) issue(p, xr[p], wr[p]);
  int i = 0;
  for (; i + R <= n16; i += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      issue(i + u + PD, xr[(u + PD) % R], wr[(u + PD) % R]);
      __builtin_amdgcn_sched_barrier(0);
      mma(xr[u], wr[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // fewer than R groups left, already loaded into sets 0 .. PD - 1
#pragma unroll
  for (int u = 0; u < PD; ++u)
    if (i + u < n16) mma(xr[u], wr[u]);
}

// Partial scores of one wavefront: token block tb, score-column blocks
// cb0 .. cb0 + NCB - 1, depth [k0, k0 + kq) (kq a multiple of 16).  Lane l
// ends with token tb*32 + l % 32 and columns cb*32 + 8 (v / 4) + 4 (l / 32)
// + v % 4 in acc[cb - cb0][v].  The next 16 k are loaded before the
// current 16 k's MFMAs (two register sets, loop unrolled by two).  FP32
// MFMAs for fp32 activations; the bf16 form above for 16-bit ones.
template <int XT, int NCB>
__device__ __forceinline__ void score_tiles(const RouteArgs& a, int tb, int cb0, int k0, int kq, int lane,
                                            f16v (&acc)[NCB]) {
  if constexpr (XT != DT_F32) {
    f16v acc1[1][NCB];
    score_tiles_bf<XT, NCB, 1>(a, tb, cb0, k0, kq, lane, acc1);
#pragma unroll
    for (int c = 0; c < NCB; ++c) acc[c] = acc1[0][c];
    return;
  }
  using XE = typename Elem<XT>::T;
  const int h = lane >> 5;
  int tok = tb * 32 + (lane & 31);
  tok = tok < a.T ? tok : a.T - 1;  // rows past the batch repeat the last one
  const XE* xp = static_cast<const XE*>(a.X) + (long)tok * a.d + k0 + 8 * h;
  const float* wp = a.Wr + ((long)(k0 / 16) * a.NCp + cb0 * 32 + (lane & 31)) * 16 + 8 * h;
  const long wstep = (long)a.NCp * 16;
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  const int n16 = kq / 16;
  if (n16 == 0) return;
  auto issue = [&](int i, float (&xv)[8], f4v (&wv)[NCB][2]) {
    const int ic = i < n16 ? i : n16 - 1;  // the last group re-reads itself
    load8x<XT>(xp + ic * 16, xv);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const float* q = wp + ic * wstep + c * 32 * 16;
      wv[c][0] = *reinterpret_cast<const f4v*>(q);
      wv[c][1] = *reinterpret_cast<const f4v*>(q + 4);
    }
  };
  auto mma = [&](const float (&xv)[8], const f4v (&wv)[NCB][2]) {
    // k steps outermost: consecutive MFMAs update different accumulators
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(wv[c][st >> 2][st & 3], xv[st], acc[c], 0, 0, 0);
  };
  // loads run PD = 2 groups of 16 k ahead of the MFMAs (a ring of three
  // register sets): one group's MFMAs are too few to cover a load's latency
  constexpr int PD = 2, R = PD + 1;
  float xr[R][8];
  f4v wr[R][NCB][2];
#pragma unroll
  for (int p = 0; p < PD; ++p) issue(p, xr[p], wr[p]);
  int i = 0;
  for (; i + R <= n16; i += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      issue(i + u + PD, xr[(u + PD) % R], wr[(u + PD) % R]);
      __builtin_amdgcn_sched_barrier(0);
      mma(xr[u], wr[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // fewer than R groups left, already loaded into sets 0 .. PD - 1
#pragma unroll
  for (int u = 0; u < PD; ++u)
    if (i + u < n16) mma(xr[u], wr[u]);
}

// grid: (token blocks of 32) x (score-column blocks of 32) x splits.  The 4
// wavefronts take consecutive quarters of the split's k range; their sums
// meet in LDS.  Output: L[split][t][NCp].
template <int XT>
__global__ __launch_bounds__(256) void logits_kernel(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) float red[4][16][64];
  const int nct = a.NCp / 32;
  const int tb = blockIdx.x % ((a.T + 31) / 32);
  const int rest = blockIdx.x / ((a.T + 31) / 32);
  const int cb = rest % nct, split = rest / nct;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int kq = a.d / (4 * a.nsplit);  // k per wavefront (multiple of 16)
  f16v acc[1];
  score_tiles<XT, 1>(a, tb, cb, (split * 4 + wave) * kq, kq, lane, acc);
#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave][v][lane] = acc[0][v];
  __syncthreads();
  // thread (vg, lane): rows 8 vg + 4 h .. +3 of the block for token lane % 32
  const int vg = threadIdx.x >> 6;
  const int t = tb * 32 + (lane & 31);
  if (t < a.T) {
    f4v o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = 4 * vg + q;
      o[q] = (red[0][v][lane] + red[1][v][lane]) + (red[2][v][lane] + red[3][v][lane]);
    }
    *reinterpret_cast<f4v*>(a.L + ((long)split * a.T + t) * a.NCp + cb * 32 + 8 * vg + 4 * h) = o;
  }
}

// ------------------------------------------------------------- select --
// Thread-per-token form (used by the fused kernel): one thread walks its
// scores (biases included): the group scores, then the chosen groups'
// expert scores, keeping the best n
// (larger score first, ties to the lower index, NaN ranked last).  With
// count_experts off the per-chunk expert counters are left alone (only the
// group lists are built).
template <int NMAX>
__device__ __forceinline__ void keep_best(float v, int i, int n, float (&bv)[NMAX], int (&bi)[NMAX]) {
  v = (v == v) ? v : -INFINITY;
  if (bi[n - 1] >= 0 && !(v > bv[n - 1])) return;
  int p = n - 1;
  while (p > 0 && (bi[p - 1] < 0 || v > bv[p - 1])) {
    bv[p] = bv[p - 1];
    bi[p] = bi[p - 1];
    --p;
  }
  bv[p] = v;
  bi[p] = i;
}

// lcg / lce (optional): LDS counters [chunk - cg0][G] and [chunk - ce0][E]
// that the caller flushes to the global per-chunk counters once per
// workgroup (one global atomic per (chunk, bin) instead of one per token).
__device__ void select_token(const RouteArgs& a, int t, const float* st, int* lcg = nullptr, int cg0 = 0,
                             int* lce = nullptr, int ce0 = 0) {
  // level 1: groups
  float gv[MAX_KG];
  int gi[MAX_KG];
  for (int q = 0; q < MAX_KG; ++q) {
    gv[q] = -INFINITY;
    gi[q] = -1;
  }
  for (int g = 0; g < a.G; ++g) keep_best<MAX_KG>(st[g], g, a.kg, gv, gi);
  float ps = 0.f;
  for (int q = 0; q < a.kg; ++q) ps += expf(gv[q] - gv[0]);
  // level 2: experts inside each chosen group, in selection order
  for (int ga = 0; ga < a.kg; ++ga) {
    const int g = gi[ga];
    const float pg = expf(gv[ga] - gv[0]) / ps;
    if (a.K == 1) {
      const int slot = t * a.k + ga;
      a.idx[slot] = g;
      a.w[slot] = pg;
      if (a.count_experts) {
        if (lce) atomicAdd(&lce[(slot / CHUNK - ce0) * a.E + g], 1);
        else atomicAdd(&a.ccount[(slot / CHUNK) * a.E + g], 1);
      }
    } else {
      float ev[MAX_SLOTS];
      int ei[MAX_SLOTS];
      for (int q = 0; q < MAX_SLOTS; ++q) {
        ev[q] = -INFINITY;
        ei[q] = -1;
      }
      const float* se = st + a.G + g * a.K;
      for (int j = 0; j < a.K; ++j) keep_best<MAX_SLOTS>(se[j], j, a.ke, ev, ei);
      float qs = 0.f;
      for (int b = 0; b < a.ke; ++b) qs += expf(ev[b] - ev[0]);
      for (int b = 0; b < a.ke; ++b) {
        const int slot = t * a.k + ga * a.ke + b;
        const int ex = g * a.K + ei[b];
        a.idx[slot] = ex;
        a.w[slot] = pg * (expf(ev[b] - ev[0]) / qs);
        if (a.count_experts) {
          if (lce) atomicAdd(&lce[(slot / CHUNK - ce0) * a.E + ex], 1);
          else atomicAdd(&a.ccount[(slot / CHUNK) * a.E + ex], 1);
        }
      }
    }
    const int gslot = t * a.kg + ga;
    a.gidx[gslot] = g;
    if (lcg) atomicAdd(&lcg[(gslot / CHUNK - cg0) * a.G + g], 1);
    else atomicAdd(&a.cgcount[(gslot / CHUNK) * a.G + g], 1);
  }
}

__device__ __forceinline__ float score_bias(const RouteArgs& a, int c) {
  if (c < a.G) return a.gbias ? a.gbias[c] : 0.f;
  return a.ebias ? a.ebias[c - a.G] : 0.f;
}

// Wavefront top-k in the order keep_best gives (higher score first, ties to
// the lower index, NaN as -inf).  Up to 64 candidates: lane c ranks
// candidate c by counting the candidates ahead of it.  More: candidate c
// sits on lane c % 64 and each round takes the best remaining one by a
// butterfly over the lanes.  Selection r ends up in lane r's (myv, myi).
// k <= n, k <= 64.
__device__ void wave_topk(const float* sv, int n, int k, int lane, float& myv, int& myi) {
  if (n <= 64) {
    // one candidate per lane, ranked against all n in that same order (a
    // total order, so the ranks are 0 .. n-1): no cross-lane rounds
    float v = -INFINITY;
    if (lane < n) {
      v = sv[lane];
      v = (v == v) ? v : -INFINITY;
    }
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      float u = sv[j];
      u = (u == u) ? u : -INFINITY;
      rank += (u > v || (u == v && j < lane)) ? 1 : 0;
    }
    myv = -INFINITY;
    myi = -1;
    for (int r = 0; r < k; ++r) {
      const unsigned long long m = __ballot(lane < n && rank == r);
      const int c = __ffsll((long long)m) - 1;
      if (lane == r) {
        float u = sv[c];
        myv = (u == u) ? u : -INFINITY;
        myi = c;
      }
    }
    return;
  }
  uint32_t used = 0;  // bit q: candidate lane + 64 q taken
  myv = -INFINITY;
  myi = -1;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    int bok = 0;
    for (int q = 0; lane + 64 * q < n; ++q) {
      if ((used >> q) & 1u) continue;
      float v = sv[lane + 64 * q];
      v = (v == v) ? v : -INFINITY;
      if (!bok || v > bv) {
        bv = v;
        bi = lane + 64 * q;
        bok = 1;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      const int ook = __shfl_xor(bok, m);
      if (ook && (!bok || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
        bok = 1;
      }
    }
    if (lane == r) {
      myv = bv;
      myi = bi;
    }
    if ((bi & 63) == lane) used |= 1u << (bi >> 6);
  }
}

// One token's two-level selection by a wavefront; the gates are
// select_token's arithmetic term by term (same sums in the same order).
__device__ void select_token_wave(const RouteArgs& a, int t, const float* st, int lane) {
  float gvl;
  int gil;
  wave_topk(st, a.G, a.kg, lane, gvl, gil);
  const float g0 = __shfl(gvl, 0);
  float ps = 0.f;
  for (int q = 0; q < a.kg; ++q) ps += expf(__shfl(gvl, q) - g0);
  for (int ga = 0; ga < a.kg; ++ga) {
    const int g = __shfl(gil, ga);
    const float pg = expf(__shfl(gvl, ga) - g0) / ps;
    if (a.K == 1) {
      const int slot = t * a.k + ga;
      if (lane == 0) {
        a.idx[slot] = g;
        a.w[slot] = pg;
        if (a.count_experts) atomicAdd(&a.ccount[(slot / CHUNK) * a.E + g], 1);
      }
    } else {
      float evl;
      int eil;
      wave_topk(st + a.G + g * a.K, a.K, a.ke, lane, evl, eil);
      const float e0 = __shfl(evl, 0);
      float qs = 0.f;
      for (int b = 0; b < a.ke; ++b) qs += expf(__shfl(evl, b) - e0);
      if (lane < a.ke) {
        const int slot = t * a.k + ga * a.ke + lane;
        const int ex = g * a.K + eil;
        a.idx[slot] = ex;
        a.w[slot] = pg * (expf(evl - e0) / qs);
        if (a.count_experts) atomicAdd(&a.ccount[(slot / CHUNK) * a.E + ex], 1);
      }
    }
    if (lane == 0) {
      const int gslot = t * a.kg + ga;
      a.gidx[gslot] = g;
      atomicAdd(&a.cgcount[(gslot / CHUNK) * a.G + g], 1);
    }
  }
}

// A workgroup takes tpb consecutive tokens: its 256 threads first sum the
// k-split partials of all their scores (plus the biases) into LDS, then
// each wavefront selects for every fourth token.
__global__ __launch_bounds__(256) void select_kernel(RouteArgs a, int tpb) {
  extern __shared__ float sc[];  // [tpb][NC]
  const int NC = a.G + (a.K > 1 ? a.G * a.K : 0);
  const int t0 = blockIdx.x * tpb;
  const int nt = min(tpb, a.T - t0);
  const long stride = (long)a.T * a.NCp;
  for (int e = threadIdx.x; e < nt * NC; e += 256) {
    const int tk = e / NC, c = e - tk * NC;
    const float* p = a.L + (long)(t0 + tk) * a.NCp + c;
    // every partial in flight at once (they were written by other
    // workgroups, often on other XCDs: one latency, not nsplit of them),
    // then summed pairwise
    float q[kMaxRouterSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxRouterSplits; ++sp) q[sp] = sp < a.nsplit ? p[sp * stride] : 0.f;
#pragma unroll
    for (int st = 1; st < kMaxRouterSplits; st <<= 1)
#pragma unroll
      for (int sp = 0; sp + st < kMaxRouterSplits; sp += 2 * st) q[sp] += q[sp + st];
    sc[e] = q[0] + score_bias(a, c);
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int tk = wave; tk < nt; tk += 4) select_token_wave(a, t0 + tk, sc + tk * NC, lane);
}

// Scores and selection in one kernel when a 32-token block's scores fit one
// workgroup (at most 4 column blocks): wavefront w of NW (4 or 8) computes k
// range w of every column block, the NW partial blocks meet in LDS
// (dynamic, summed pairwise in a fixed order), and one thread per token
// selects.  More wavefronts shorten the dependent MFMA chain of the few
// workgroups a small batch has.  For large batches of 16-bit activations a
// workgroup takes TBN = 2 token blocks, which share the loads of the router
// matrix parts (their partial blocks go through LDS one block at a time).
template <int XT, int NCB, int NW, int TBN = 1>
__global__ __launch_bounds__(64 * NW) void route_fused_kernel(RouteArgs a) {
  static_assert(TBN == 1 || XT != DT_F32, "several token blocks: 16-bit activations only");
  extern __shared__ __attribute__((aligned(16))) float red[];  // [NW][NCB][16][64]
  __shared__ float sc[32 * TBN][NCB * 32 + 1];
  // per-workgroup routing counts: 32 TBN tokens span at most TBN + 1
  // group-list chunks and 2 TBN + 1 expert-list chunks of 256 assignments
  // (at most 8 groups and 16 experts per token)
  __shared__ int lcg[(TBN + 1) * 256];
  __shared__ int lce[(2 * TBN + 1) * 1024];
  const int tb = blockIdx.x * TBN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int NT = 64 * NW;
  const int kq = a.d / NW;
  for (int i = threadIdx.x; i < (TBN + 1) * a.G; i += NT) lcg[i] = 0;
  if (a.count_experts)
    for (int i = threadIdx.x; i < (2 * TBN + 1) * a.E; i += NT) lce[i] = 0;
  const int NC = a.G + (a.K > 1 ? a.G * a.K : 0);
  f16v acc[TBN][NCB];
  if constexpr (XT != DT_F32) {
    score_tiles_bf<XT, NCB, TBN>(a, tb, 0, wave * kq, kq, lane, acc);
  } else {
    score_tiles<XT, NCB>(a, tb, 0, wave * kq, kq, lane, acc[0]);
  }
#pragma unroll
  for (int b = 0; b < TBN; ++b) {
    if (b > 0) __syncthreads();  // the previous block's partials are summed
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((wave * NCB + cb) * 16 + v) * 64 + lane] = acc[b][cb][v];
    __syncthreads();
    for (int e = threadIdx.x; e < NCB * 16 * 64; e += NT) {
      const int cb = e / (16 * 64), v = (e / 64) % 16, l = e % 64;
      const int c = cb * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
      if (c < NC) {
        // pairwise over the wavefronts' partials
        float p[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) p[w] = red[w * NCB * 16 * 64 + e];
#pragma unroll
        for (int st = 1; st < NW; st <<= 1)
#pragma unroll
          for (int w = 0; w + st < NW; w += 2 * st) p[w] += p[w + st];
        sc[b * 32 + (l & 31)][c] = p[0] + score_bias(a, c);
      }
    }
  }
  __syncthreads();
  const int t = tb * 32 + threadIdx.x;
  const int t0 = tb * 32;
  const int cg0 = t0 * a.kg / CHUNK, ce0 = t0 * a.k / CHUNK;
  if (threadIdx.x < 32 * TBN && t < a.T) select_token(a, t, sc[threadIdx.x], lcg, cg0, lce, ce0);
  __syncthreads();
  for (int i = threadIdx.x; i < (TBN + 1) * a.G; i += NT)
    if (lcg[i]) atomicAdd(&a.cgcount[(cg0 + i / a.G) * a.G + i % a.G], lcg[i]);
  if (a.count_experts)
    for (int i = threadIdx.x; i < (2 * TBN + 1) * a.E; i += NT)
      if (lce[i]) atomicAdd(&a.ccount[(ce0 + i / a.E) * a.E + i % a.E], lce[i]);
}

// Exclusive scan of n (<= 1024) ints held in lds_in into lds_out[0..n];
// 256 threads, each owning 4 consecutive entries.
__device__ void block_exscan(const int* lds_in, int* lds_out, int n, int* tmp) {
  const int tid = threadIdx.x;
  int v[4], s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int i = tid * 4 + j;
    v[j] = (i < n) ? lds_in[i] : 0;
    s += v[j];
  }
  tmp[tid] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int add = (tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  int run = tmp[tid] - s;  // exclusive prefix of this thread's 4 entries
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int i = tid * 4 + j;
    if (i < n) lds_out[i] = run;
    run += v[j];
  }
  if (tid == 255) lds_out[n] = tmp[255];
  __syncthreads();
}

// One level (experts or groups) of the stable scatter for chunk b.
// lds needs 7 * nbins + 257 ints.
__device__ void bin_scatter(int b, int n_assign, int slots, int nbins, const int* assign,
                            const int* chunk_counts, int nch, int* counts_out, int* offsets_out,
                            int* perm_tok, int* perm_aid, int* lds) {
  int* tot = lds;                 // [nbins]
  int* bef = tot + nbins;         // [nbins]
  int* off = bef + nbins;         // [nbins + 1]
  int* wcnt = off + nbins + 1;    // [4][nbins]
  int* tmp = wcnt + 4 * nbins;    // [256]
  const int tid = threadIdx.x;
  for (int e = tid; e < nbins; e += 256) {
    tot[e] = 0;
    bef[e] = 0;
    wcnt[e] = wcnt[nbins + e] = wcnt[2 * nbins + e] = wcnt[3 * nbins + e] = 0;
  }
  __syncthreads();
  for (int pidx = tid; pidx < nch * nbins; pidx += 256) {
    const int c = pidx / nbins, e = pidx - c * nbins;
    const int v = chunk_counts[pidx];
    if (v) {
      atomicAdd(&tot[e], v);
      if (c < b) atomicAdd(&bef[e], v);
    }
  }
  __syncthreads();
  block_exscan(tot, off, nbins, tmp);
  if (b == 0) {
    for (int e = tid; e < nbins; e += 256) counts_out[e] = tot[e];
    for (int e = tid; e <= nbins; e += 256) offsets_out[e] = off[e];
  }
  // rank of each assignment among equal bins earlier in its wave
  const int aid = b * CHUNK + tid;
  const bool valid = aid < n_assign;
  const int e = valid ? assign[aid] : -1;
  const int lane = tid & 63, wv = tid >> 6;
  int rank = 0;
  bool pending = valid;
  while (true) {
    const unsigned long long act = __ballot(pending);
    if (act == 0ull) break;
    const int leader = __ffsll(act) - 1;
    const int ee = __shfl(e, leader);
    const bool hit = pending && e == ee;
    const unsigned long long m = __ballot(hit);
    if (hit) {
      rank = __popcll(m & ((1ull << lane) - 1ull));
      pending = false;
    }
    if (lane == 0) wcnt[wv * nbins + ee] = __popcll(m);
  }
  __syncthreads();
  if (valid) {
    int pos = off[e] + bef[e] + rank;
    for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2 * nbins + e];
    if (perm_tok) perm_tok[pos] = aid / slots;
    if (perm_aid) perm_aid[pos] = aid;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  extern __shared__ int lds[];
  const int b = blockIdx.x;
  // with no assignments block 0 still publishes zero counts and offsets
  if (a.do_experts && b < (a.nch_e > 0 ? a.nch_e : 1))
    bin_scatter(b, a.T * a.k, a.k, a.E, a.idx, a.ccount, a.nch_e, a.counts, a.offsets, a.perm,
                nullptr, lds);
  if (b < (a.nch_g > 0 ? a.nch_g : 1))
    bin_scatter(b, a.T * a.kg, a.kg, a.G, a.gidx, a.cgcount, a.nch_g, a.gcounts, a.goffsets,
                a.gperm, a.garow, lds);
}

__global__ void zero_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

template <int XT>
hipError_t launch_logits(const RouteArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((a.T + 31) / 32) * (a.NCp / 32) * a.nsplit;
  hipLaunchKernelGGL(logits_kernel<XT>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int XT, int NCB, int NW, int TBN = 1>
hipError_t launch_fused_nw(const RouteArgs& a, hipStream_t st) {
  auto k = route_fused_kernel<XT, NCB, NW, TBN>;
  const size_t lds = (size_t)NW * NCB * 16 * 64 * sizeof(float);
  if (lds > 65536 || TBN > 1) {  // (TBN > 1: over 64 KB with the static arrays)
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3((a.T + 32 * TBN - 1) / (32 * TBN)), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

// Wavefronts per workgroup: 8 when the batch has fewer 32-token blocks than
// the chip has compute units (the chain length then decides) and each
// wavefront still keeps at least 128 of the d products; else 4, which
// leaves more LDS for other workgroups on the same compute unit.
inline int fused_waves(int T, int d) {
  return ((T + 31) / 32 < 256 && d % (16 * 8) == 0 && d / 8 >= 128) ? 8 : 4;
}

template <int XT, int NCB>
hipError_t launch_fused_ncb(const RouteArgs& a, hipStream_t st) {
  if (fused_waves(a.T, a.d) == 8) return launch_fused_nw<XT, NCB, 8>(a, st);
  // two token blocks per workgroup once that still gives a workgroup per
  // compute unit (up to 3 column blocks: 4 would spill)
  if constexpr (XT != DT_F32 && NCB <= 3) {
    if ((a.T + 63) / 64 >= 256) return launch_fused_nw<XT, NCB, 4, 2>(a, st);
  }
  return launch_fused_nw<XT, NCB, 4>(a, st);
}

template <int XT>
hipError_t launch_fused(const RouteArgs& a, int ncb, hipStream_t st) {
  switch (ncb) {
    case 1: return launch_fused_ncb<XT, 1>(a, st);
    case 2: return launch_fused_ncb<XT, 2>(a, st);
    case 3: return launch_fused_ncb<XT, 3>(a, st);
    case 4: return launch_fused_ncb<XT, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_router(int x_dtype, const RouteArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
  const int ncb = a.NCp / 32;
  if (a.nsplit == 1 && ncb <= 4) {
    switch (x_dtype) {
      case DT_F32: return launch_fused<DT_F32>(a, ncb, st);
      case DT_F16: return launch_fused<DT_F16>(a, ncb, st);
      case DT_BF16: return launch_fused<DT_BF16>(a, ncb, st);
    }
    return e;
  }
  switch (x_dtype) {
    case DT_F32: e = launch_logits<DT_F32>(a, st); break;
    case DT_F16: e = launch_logits<DT_F16>(a, st); break;
    case DT_BF16: e = launch_logits<DT_BF16>(a, st); break;
  }
  if (e != hipSuccess) return e;
  // tokens per selection workgroup: about 64 workgroups for small batches,
  // at most 64 tokens and 64 KiB of scores each
  const int NC = a.G + (a.K > 1 ? a.G * a.K : 0);
  int tpb = 1;
  while (tpb < 64 && (long)a.T >= 64L * 2 * tpb && (size_t)2 * tpb * NC * sizeof(float) <= 65536) tpb *= 2;
  const size_t lds = (size_t)tpb * NC * sizeof(float);
  hipLaunchKernelGGL(select_kernel, dim3((a.T + tpb - 1) / tpb), dim3(256), lds, st, a, tpb);
  return hipGetLastError();
}

// k splits of the router GEMM: enough workgroups for the chip, each
// wavefront keeping at least 64 of the d products.
int router_splits(int T, int d, int NCp) {
  if (NCp <= 128) return 1;  // scores and selection fused
  const long blocks = (long)((T + 31) / 32) * (NCp / 32);
  int s = 1;
  while (s < kMaxRouterSplits && blocks * s < 256 && d % (4 * 16 * 2 * s) == 0 && d / (4 * 2 * s) >= 64) s *= 2;
  return s;
}

// Counting sort of group g's rows by the Gray-code rank of the 8-bit fold
// of their expert set (the same key the input projection's tile sort uses;
// for groups of at most 8 experts the fold is the set itself, and
// neighbouring keys are sets that differ by one expert).  Rows of equal key
// keep no particular order: each token's results depend only on its own
// row, so the order changes no value, and a 32-row block of the sorted list
// then sees few distinct experts.  Keys are computed once, eight rows per
// thread at a time (their loads in flight together), and kept in LDS when
// the group fits (kcap bytes), else recomputed; both passes take B rows per
// thread at a time with all their global loads issued before any LDS update.
__device__ __forceinline__ int group_row_key(const GroupSortArgs& a, int g, int aid) {
  const int t = aid / a.kg, ga = aid - t * a.kg;
  const int* ip = a.idx + t * a.k + ga * a.ke;
  uint64_t set = 0;
#pragma unroll
  for (int s = 0; s < MAX_SLOTS; ++s)
    if (s < a.ke) set |= 1ull << (ip[s] - g * a.K);
  uint32_t f = static_cast<uint32_t>(set) ^ static_cast<uint32_t>(set >> 32);
  f ^= f >> 16;
  f ^= f >> 8;
  return static_cast<int>(gray_rank8(f & 255u));
}

__global__ __launch_bounds__(256) void group_sort_kernel(GroupSortArgs a, int kcap) {
  extern __shared__ uint8_t skey[];  // [kcap]
  __shared__ int hist[256];
  __shared__ int cur[256];
  __shared__ int wsum[4];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = a.goffsets[g], n = a.goffsets[g + 1] - r0;
  const bool keep = n <= kcap;
  hist[tid] = 0;
  __syncthreads();
  constexpr int B = 8;
  for (int i0 = 0; i0 < n; i0 += 256 * B) {
    int aid[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = i0 + b * 256 + tid;
      aid[b] = i < n ? a.garow_in[r0 + i] : -1;
    }
    // all B rows' expert loads in flight before any LDS update
    int key[B];
#pragma unroll
    for (int b = 0; b < B; ++b) key[b] = aid[b] < 0 ? -1 : group_row_key(a, g, aid[b]);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (key[b] < 0) continue;
      atomicAdd(&hist[key[b]], 1);
      if (keep) skey[i0 + b * 256 + tid] = static_cast<uint8_t>(key[b]);
    }
  }
  __syncthreads();
  // exclusive scan of the 256 bins
  const int cnt = hist[tid];
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  cur[tid] = base + inc - cnt;
  __syncthreads();
  for (int i0 = 0; i0 < n; i0 += 256 * B) {
    int aid[B], key[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = i0 + b * 256 + tid;
      aid[b] = i < n ? a.garow_in[r0 + i] : -1;
    }
#pragma unroll
    for (int b = 0; b < B; ++b)
      key[b] = aid[b] < 0 ? -1 : (keep ? static_cast<int>(skey[i0 + b * 256 + tid]) : group_row_key(a, g, aid[b]));
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (key[b] >= 0) a.garow_out[r0 + atomicAdd(&cur[key[b]], 1)] = aid[b];
  }
}

hipError_t launch_group_sort(const GroupSortArgs& a, int max_rows, hipStream_t st) {
  if (a.G <= 0) return hipSuccess;
  const int kcap = max_rows < 32768 ? max_rows : 32768;
  hipLaunchKernelGGL(group_sort_kernel, dim3(a.G), dim3(256), (size_t)kcap, st, a, kcap);
  return hipGetLastError();
}

size_t scatter_lds_bytes(int E, int G) {
  int nb = E > G ? E : G;
  return sizeof(int) * (7 * (size_t)nb + 257 + 8);
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t st) {
  int nblk = (a.do_experts && a.nch_e > a.nch_g) ? a.nch_e : a.nch_g;
  if (nblk <= 0) nblk = 1;  // T == 0 still publishes zero counts and offsets
  hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(256), scatter_lds_bytes(a.E, a.G), st, a);
  return hipGetLastError();
}

hipError_t launch_zero(int* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace cefn
