// Routing kernels: two-level top-k router and the stable per-bin token lists.
//
// Router ("Breaking the MoE LLM Trilemma", papernotes.org note, key design 3:
// groups first, then experts inside the chosen groups; FP32 router as in the
// MoE routing page "混合专家模型的路由机制与工程落地", section 3.1): 64-lane
// wavefronts, each routing one to four tokens.  Lanes split the model width,
// partial dot products are combined with cross-lane xor reductions, and the
// top-k keeps the larger score, then the lower index.
//
// Token lists (dropless dispatch, tokens ascending within each bin): the
// router counts assignments per (chunk of 256 assignments, bin) with
// atomics; the scatter kernel turns those counts into per-bin offsets with a
// prefix sum and places each assignment at offset + (assignments of the same
// bin in earlier chunks) + (its rank inside its own chunk), the rank coming
// from a wave ballot over equal bins, so the result does not depend on
// scheduling.
#include "common.h"
#include "kernels.h"

namespace cefn {

namespace {

__device__ __forceinline__ int next_pow2(int c) {
  int p = 1;
  while (p < c) p <<= 1;
  return p;
}

// Logits x . W[:, c] for c < C (W row stride ldw).  Lane l ends up holding
// column l + 64 q in out[q] (columns >= C hold garbage).
template <int XT, int NQ>
__device__ void wave_logits(const typename Elem<XT>::T* x, int d, const float* W, int ldw, int C,
                            int lane, float (&out)[NQ]) {
  if (C <= 64) {
    const int Cp = next_pow2(C);
    const int S = 64 / Cp;
    const int col = lane & (Cp - 1);
    const int sl = lane / Cp;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if (col < C) {
      int i = sl;
      for (; i + 3 * S < d; i += 4 * S) {
        a0 = fmaf(load_as_f32<XT>(x, i), W[(long)i * ldw + col], a0);
        a1 = fmaf(load_as_f32<XT>(x, i + S), W[(long)(i + S) * ldw + col], a1);
        a2 = fmaf(load_as_f32<XT>(x, i + 2 * S), W[(long)(i + 2 * S) * ldw + col], a2);
        a3 = fmaf(load_as_f32<XT>(x, i + 3 * S), W[(long)(i + 3 * S) * ldw + col], a3);
      }
      for (; i < d; i += S) a0 = fmaf(load_as_f32<XT>(x, i), W[(long)i * ldw + col], a0);
    }
    float acc = (a0 + a1) + (a2 + a3);
    for (int off = Cp; off < 64; off <<= 1) acc += __shfl_xor(acc, off);
    out[0] = acc;
#pragma unroll
    for (int q = 1; q < NQ; ++q) out[q] = 0.f;
  } else {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = lane + 64 * q;
      float a0 = 0.f, a1 = 0.f;
      if (c < C) {
        int i = 0;
        for (; i + 1 < d; i += 2) {
          a0 = fmaf(load_as_f32<XT>(x, i), W[(long)i * ldw + c], a0);
          a1 = fmaf(load_as_f32<XT>(x, i + 1), W[(long)(i + 1) * ldw + c], a1);
        }
        for (; i < d; ++i) a0 = fmaf(load_as_f32<XT>(x, i), W[(long)i * ldw + c], a0);
      }
      out[q] = a0 + a1;
    }
  }
}

// k largest of the C values spread as in wave_logits; ties to the lower
// column.  sel/val receive columns and values, best first (wave-uniform).
template <int NQ, int KMAX>
__device__ void wave_topk(const float (&v)[NQ], int C, int k, int lane, int (&sel)[KMAX],
                          float (&val)[KMAX]) {
  bool taken[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) taken[q] = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int c = lane + 64 * q;
        // a NaN score ranks as -inf, so every untaken column stays a
        // candidate and the result is always a valid column
        const float vq = (v[q] == v[q]) ? v[q] : -INFINITY;
        if (c < C && !taken[q] && (vq > bv || (vq == bv && c < bi))) {
          bv = vq;
          bi = c;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        float ov = __shfl_xor(bv, off);
        int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sel[j] = bi;
      val[j] = bv;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + 64 * q == bi) taken[q] = true;
    } else {
      sel[j] = 0;
      val[j] = 0.f;
    }
  }
}

template <int KMAX>
__device__ void softmax_sel(const float (&val)[KMAX], int k, float (&p)[KMAX]) {
  float m = val[0];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    p[j] = (j < k) ? expf(val[j] - m) : 0.f;
    s += p[j];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) p[j] = p[j] / s;
}

template <int XT>
__global__ __launch_bounds__(256) void router_generic_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  using XE = typename Elem<XT>::T;
  const XE* x = static_cast<const XE*>(a.X) + (long)t * a.d;

  // level 1: groups
  float s[4];
  wave_logits<XT, 4>(x, a.d, a.Wg, a.G, a.G, lane, s);
  if (a.gbias) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = lane + 64 * q;
      if (c < a.G) s[q] += a.gbias[c];
    }
  }
  int gsel[MAX_KG];
  float gval[MAX_KG], p[MAX_KG];
  wave_topk<4, MAX_KG>(s, a.G, a.kg, lane, gsel, gval);
  softmax_sel<MAX_KG>(gval, a.kg, p);

  // level 2: experts inside each chosen group
#pragma unroll
  for (int ga = 0; ga < MAX_KG; ++ga) {
    if (ga >= a.kg) break;
    const int g = gsel[ga];
    if (a.K == 1) {
      if (lane == 0) {
        const int slot = t * a.k + ga;
        a.idx[slot] = g;
        a.w[slot] = p[ga];
        atomicAdd(&a.ccount[(slot / CHUNK) * a.E + g], 1);
      }
    } else {
      float e[4];
      wave_logits<XT, 4>(x, a.d, a.We + (long)g * a.d * a.K, a.K, a.K, lane, e);
      if (a.ebias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int c = lane + 64 * q;
          if (c < a.K) e[q] += a.ebias[g * a.K + c];
        }
      }
      int jsel[MAX_SLOTS];
      float jval[MAX_SLOTS], q[MAX_SLOTS];
      wave_topk<4, MAX_SLOTS>(e, a.K, a.ke, lane, jsel, jval);
      softmax_sel<MAX_SLOTS>(jval, a.ke, q);
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < MAX_SLOTS; ++b) {
          if (b >= a.ke) break;
          const int slot = t * a.k + ga * a.ke + b;
          const int ex = g * a.K + jsel[b];
          a.idx[slot] = ex;
          a.w[slot] = p[ga] * q[b];
          atomicAdd(&a.ccount[(slot / CHUNK) * a.E + ex], 1);
        }
      }
    }
    if (lane == 0) {
      const int gslot = t * a.kg + ga;
      a.gidx[gslot] = g;
      atomicAdd(&a.cgcount[(gslot / CHUNK) * a.G + g], 1);
    }
  }
}


// ---------------------------------------------------------------------------
// Router for the common shapes (G and K fixed at compile time, each a
// multiple of 4 up to 16, or K = 1).  Wavefront w routes TPW tokens
// together.  Lane l owns rows 4 (l + 64 m) .. +3 of d (m < d / 256) and
// loads them as vectors: 4 activations per token and 4 rows of the router
// matrix (row-major, so 4 * C consecutive floats, read as 16-byte vectors).
// The group-level pass shares every weight load among the TPW tokens; the
// expert-level pass runs once per (token, chosen group).  The loops carry no
// branches, so the loads of a step are all in flight together.  One xor
// butterfly per logit leaves every lane holding every logit, so the top-k
// and the softmax run per lane without further cross-lane traffic.
template <int XT>
__device__ __forceinline__ void load4(const typename Elem<XT>::T* p, float (&v)[4]) {
  if constexpr (XT == DT_F32) {
    f4v q = *reinterpret_cast<const f4v*>(p);
    v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
  } else {
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    u2v q = *reinterpret_cast<const u2v*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t b = static_cast<uint16_t>((q[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      v[e] = (XT == DT_F16) ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
    }
  }
}

// acc[p][c] = sum over d of x_p[i] W[i][c] for NT token rows and the C
// columns of W (row stride C); totals end up in every lane.
template <int XT, int NT, int C>
__device__ __forceinline__ void dot_pass(const typename Elem<XT>::T* const (&xs)[NT],
                                         const float* W, int d, int lane, float (&acc)[NT][C]) {
#pragma unroll
  for (int p = 0; p < NT; ++p)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[p][c] = 0.f;
  const int steps = d / 256;
#pragma unroll 2
  for (int m = 0; m < steps; ++m) {
    const int i0 = 4 * (lane + 64 * m);
    float x[NT][4];
#pragma unroll
    for (int p = 0; p < NT; ++p) load4<XT>(xs[p] + i0, x[p]);
    f4v wv[4][C / 4];
    const float* w = W + (long)i0 * C;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c4 = 0; c4 < C / 4; ++c4) wv[e][c4] = *reinterpret_cast<const f4v*>(w + e * C + 4 * c4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c4 = 0; c4 < C / 4; ++c4)
#pragma unroll
        for (int p = 0; p < NT; ++p)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) acc[p][4 * c4 + cc] = fmaf(x[p][e], wv[e][c4][cc], acc[p][4 * c4 + cc]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1)
#pragma unroll
    for (int p = 0; p < NT; ++p)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[p][c] += __shfl_xor(acc[p][c], off);
}

// k best of v[0..C) (descending, ties to the lower index), in every lane.
template <int C, int KMAX>
__device__ __forceinline__ void topk_local(const float (&v)[C], int k, int (&sel)[KMAX],
                                           float (&val)[KMAX]) {
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float x = (v[c] == v[c]) ? v[c] : -INFINITY;  // NaN ranks as -inf
      if (!((taken >> c) & 1u) && (bi < 0 || x > bv)) {
        bv = x;
        bi = c;
      }
    }
    if (j < k) {
      sel[j] = bi;
      val[j] = bv;
      taken |= 1u << bi;
    } else {
      sel[j] = 0;
      val[j] = 0.f;
    }
  }
}

template <int XT, int TPW, int CG, int CK>
__global__ __launch_bounds__(256) void router_fast_kernel(RouteArgs a) {
  using XE = typename Elem<XT>::T;
  const int lane = threadIdx.x & 63;
  const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  if (t0 >= a.T) return;
  const int nt = min(TPW, a.T - t0);
  const XE* X = static_cast<const XE*>(a.X);
  const XE* xs[TPW];
#pragma unroll
  for (int p = 0; p < TPW; ++p) xs[p] = X + (long)(t0 + (p < nt ? p : 0)) * a.d;

  // level 1: group logits, one weight load shared by the TPW tokens
  float s[TPW][CG];
  dot_pass<XT, TPW, CG>(xs, a.Wg, a.d, lane, s);
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    if (p >= nt) break;
    const int t = t0 + p;
    if (a.gbias) {
#pragma unroll
      for (int c = 0; c < CG; ++c) s[p][c] += a.gbias[c];
    }
    int gsel[MAX_KG];
    float gval[MAX_KG], pg[MAX_KG];
    topk_local<CG, MAX_KG>(s[p], a.kg, gsel, gval);
    softmax_sel<MAX_KG>(gval, a.kg, pg);
    // level 2: expert logits of each chosen group
#pragma unroll
    for (int ga = 0; ga < MAX_KG; ++ga) {
      if (ga >= a.kg) break;
      const int g = gsel[ga];
      if constexpr (CK == 1) {
        if (lane == 0) {
          const int slot = t * a.k + ga;
          a.idx[slot] = g;
          a.w[slot] = pg[ga];
          atomicAdd(&a.ccount[(slot / CHUNK) * a.E + g], 1);
        }
      } else {
        const XE* x1[1] = {xs[p]};
        float e[1][CK];
        dot_pass<XT, 1, CK>(x1, a.We + (long)g * a.d * CK, a.d, lane, e);
        if (a.ebias) {
#pragma unroll
          for (int c = 0; c < CK; ++c) e[0][c] += a.ebias[g * CK + c];
        }
        int js[MAX_SLOTS];
        float jv[MAX_SLOTS], qw[MAX_SLOTS];
        topk_local<CK, MAX_SLOTS>(e[0], a.ke, js, jv);
        softmax_sel<MAX_SLOTS>(jv, a.ke, qw);
        if (lane == 0) {
#pragma unroll
          for (int b = 0; b < MAX_SLOTS; ++b) {
            if (b >= a.ke) break;
            const int slot = t * a.k + ga * a.ke + b;
            const int ex = g * CK + js[b];
            a.idx[slot] = ex;
            a.w[slot] = pg[ga] * qw[b];
            atomicAdd(&a.ccount[(slot / CHUNK) * a.E + ex], 1);
          }
        }
      }
      if (lane == 0) {
        const int gslot = t * a.kg + ga;
        a.gidx[gslot] = g;
        atomicAdd(&a.cgcount[(gslot / CHUNK) * a.G + g], 1);
      }
    }
  }
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
  if (b < (a.nch_e > 0 ? a.nch_e : 1))
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

template <int XT, int TPW, int CG, int CK>
hipError_t launch_fast(const RouteArgs& a, hipStream_t st) {
  const int waves = (a.T + TPW - 1) / TPW;
  hipLaunchKernelGGL((router_fast_kernel<XT, TPW, CG, CK>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int XT, int CG, int CK>
hipError_t launch_tpw(const RouteArgs& a, hipStream_t st) {
  // several tokens per wavefront once there are enough tokens to fill the chip
  if (a.T >= 8192) return launch_fast<XT, 4, CG, CK>(a, st);
  if (a.T >= 2048) return launch_fast<XT, 2, CG, CK>(a, st);
  return launch_fast<XT, 1, CG, CK>(a, st);
}

template <int XT>
hipError_t launch_router_t(const RouteArgs& a, hipStream_t st) {
  if (a.d % 256 == 0) {
    const int key = a.G * 100 + a.K;
    switch (key) {
      case 404: return launch_tpw<XT, 4, 4>(a, st);
      case 808: return launch_tpw<XT, 8, 8>(a, st);
      case 1616: return launch_tpw<XT, 16, 16>(a, st);
      case 401: return launch_tpw<XT, 4, 1>(a, st);
      case 801: return launch_tpw<XT, 8, 1>(a, st);
      case 1601: return launch_tpw<XT, 16, 1>(a, st);
      default: break;
    }
  }
  hipLaunchKernelGGL(router_generic_kernel<XT>, dim3((a.T + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_router(int x_dtype, const RouteArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  switch (x_dtype) {
    case DT_F32: return launch_router_t<DT_F32>(a, st);
    case DT_F16: return launch_router_t<DT_F16>(a, st);
    case DT_BF16: return launch_router_t<DT_BF16>(a, st);
  }
  return hipErrorInvalidValue;
}

size_t scatter_lds_bytes(int E, int G) {
  int nb = E > G ? E : G;
  return sizeof(int) * (7 * (size_t)nb + 257 + 8);
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t st) {
  int nblk = a.nch_e > a.nch_g ? a.nch_e : a.nch_g;
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
