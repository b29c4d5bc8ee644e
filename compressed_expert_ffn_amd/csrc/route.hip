// Routing kernels: two-level top-k router and the stable per-bin token lists.
//
// Router ("Breaking the MoE LLM Trilemma", papernotes.org note, key design 3:
// groups first, then experts inside the chosen groups; FP32 router as in the
// MoE routing page "混合专家模型的路由机制与工程落地", section 3.1): one 64-lane
// wavefront per token.  Lanes split the logit columns and the model width,
// partial dot products are combined with cross-lane xor reductions, and the
// top-k is a repeated wave arg-max (larger value, then lower index).
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
__global__ __launch_bounds__(256) void router_kernel(RouteArgs a) {
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

hipError_t launch_router(int x_dtype, const RouteArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  dim3 grid((a.T + 3) / 4), block(256);
  switch (x_dtype) {
    case DT_F32: hipLaunchKernelGGL(router_kernel<DT_F32>, grid, block, 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(router_kernel<DT_F16>, grid, block, 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL(router_kernel<DT_BF16>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
