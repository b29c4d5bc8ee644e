// Backward pass of the compressed-expert layer ("Breaking the MoE LLM
// Trilemma", papernotes.org note: the loss function / training strategy
// section trains the layer end to end; key design 2 stores each expert as
// W_base^g + A_i B_i^T).
//
// The gradient keeps the shared-base algebra of the forward pass.  With
// z_j = x W1_base + (x A1_j) B1_j^T, h_j = act(z_j) and
// y = sum_j w_j h_j W2_base + sum_j (w_j h_j A2_j) B2_j^T:
//   D     = dY W2_base^T               once per (token, group)   [rows x f]
//   e_j   = dY B2_j                    per chosen expert          [r]
//   dh_j  = w_j (D + e_j A2_j^T)       (rank-r expansion on the ALUs)
//   dz_j  = act'(z_j) dh_j,  dZbar = sum_j dz_j
//   dX    = dZbar W1_base^T + sum_j (dz_j B1_j) A1_j^T + router terms
//   dW1_base^g = X_g^T dZbar_g,   dW2_base^g = hbar_g^T dY_g
//   dA1_j = X^T (dz_j B1_j),  dB1_j = dz_j^T (x A1_j),
//   dA2_j = (w_j h_j)^T e_j,  dB2_j = dY^T (w_j h_j A2_j)
// and dw_j = <D, h_j> + <e_j, h_j A2_j> feeds the softmax backward of the
// gate.  Every GEMM here is one MFMA kernel over k-major operands (rows
// gathered on load, or k ranges that are segments of transposed, gathered
// rows); the elementwise steps run per row and per token.
#include "common.h"
#include "tile.h"
#include "train.h"

namespace cefn {
namespace {

// ------------------------------------------------------------ segment GEMM --
// A workgroup computes a 128 x 128 tile of C as 2 x 2 wavefronts of
// 64 x 64 (2 x 2 blocks of 32 x 32); both operands go straight from memory
// into registers one 64-deep stage ahead (the tile engine's direct main loop).
constexpr int BT = 128;

template <int SRC, int TY>
struct BOperand {
  using TD = TDirect<SRC, TY, 2>;
  using Raw = typename TD::Raw;
  TD td;
  struct Src {
    __device__ FragT<TY> decode(const Raw& r, int, int, int) const { return cvt_frag<SRC, TY>(r); }
  } src;
  __device__ void fetch(int kt, int, Raw (&r)[2][4]) const { td.fetch(kt, r); }
};

template <int TY, int SA>
__global__ void __launch_bounds__(256) bgemm_kernel(BGemmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int NT = (a.N + BT - 1) / BT;
  int s = 0, m0 = 0, M = 0, K = 0, n0 = 0;
  long crow0 = 0, kofs = 0;
  if (a.mode == 0) {
    // walk the segments' row tiles (S <= 256)
    int i = blockIdx.x;
    n0 = (i % NT) * BT;
    i /= NT;
    bool found = false;
    for (int q = 0; q < a.S; ++q) {
      const int cnt = a.seg_count[q];
      const int mt = (cnt + BT - 1) / BT;
      if (i < mt) {
        s = q;
        m0 = i * BT;
        M = cnt;
        found = true;
        break;
      }
      i -= mt;
    }
    if (!found) return;
    K = a.K;
    crow0 = a.seg_start[s];
  } else {
    const int MT = (a.M + BT - 1) / BT;
    int i = blockIdx.x;
    n0 = (i % NT) * BT;
    i /= NT;
    m0 = (i % MT) * BT;
    s = i / MT;
    if (s >= a.S) return;
    M = a.M;
    kofs = a.kpad_off[s];
    K = a.kpad_off[s + 1] - a.kpad_off[s];
  }
  f16v acc[2][2];
  zero_acc<2, 2>(acc);
  const int KT = K / KB;
  if (KT > 0) {
    TDirect<SA, TY, 2> to;
    const TE<SA>* abase = static_cast<const TE<SA>*>(a.a) + kofs;
    to.init(abase, a.lda, lane, [&](int t) -> long {
      const int m = m0 + wm * 64 + t * 32 + (lane & 31);
      if (m >= M) return -1;
      if (a.mode == 1) return m;
      const long pos = crow0 + m;
      return a.a_map ? (long)(a.a_map[pos] / a.a_div) : pos;
    });
    BOperand<TY, TY> bo;
    const TE<TY>* bbase = static_cast<const TE<TY>*>(a.b) + (a.mode == 0 ? (long)s * a.b_sstride : kofs);
    bo.td.init(bbase, a.ldb, lane, [&](int c) -> long {
      const int n = n0 + wn * 64 + c * 32 + (lane & 31);
      return n < a.N ? n : -1;
    });
    Mainloop<TY, 2, 2, TDirect<SA, TY, 2>, BOperand<TY, TY>, 1> ml{to, bo, lane};
    ml.template run<typename TDirect<SA, TY, 2>::Raw[2][4], typename BOperand<TY, TY>::Raw[2][4]>(KT, acc);
  }
  float* cbase = a.c + (a.mode == 0 ? crow0 * a.ldc : (long)s * a.c_sstride);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = m0 + wm * 64 + t * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int n = n0 + wn * 64 + c * 32 + acc32_row(v, lane);
        if (n < a.n_store) cbase[(long)m * a.ldc + n] = acc[t][c][v];
      }
  }
}

// ------------------------------------------------- gather + transpose ------
// One block per 64 k-columns (a padded slice of one segment) x 64 output
// rows; reads 64 source rows, writes 64 k-contiguous runs.
template <int TY, int SI>
__global__ void __launch_bounds__(256) gather_t_kernel(TransArgs a) {
  __shared__ float tileS[64][65];
  const int kc = blockIdx.x * 64;  // global padded k
  const int c0 = blockIdx.y * 64;  // output row block
  const int total = a.kpad_off[a.S];
  if (kc >= total) return;
  // segment of this k slice
  int s = 0;
  while (s + 1 < a.S && a.kpad_off[s + 1] <= kc) ++s;
  const int r0 = kc - a.kpad_off[s];
  const int cnt = a.count[s];
  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;  // source row r0 + rr, column c0 + cc
    float v = 0.f;
    if (r0 + rr < cnt && c0 + cc < a.ncols) {
      const long pos = (long)a.start[s] + r0 + rr;
      const long row = a.in_map ? (long)(a.in_map[pos] / a.in_div) : pos;
      v = load_as_f32<SI>(static_cast<const TE<SI>*>(a.in), row * a.ld_in + a.c0 + c0 + cc);
    }
    tileS[rr][cc] = v;
  }
  __syncthreads();
  TE<TY>* out = static_cast<TE<TY>*>(a.out);
  for (int i = tid; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    if (c0 + cc < a.ncols) out[(long)(c0 + cc) * a.ld_out + kc + rr] = from_f32<TY>(tileS[rr][cc]);
  }
}

__global__ void pad_scan_kernel(const int* count, int S, int* off) {
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int s = 0; s < S; ++s) {
      off[s] = acc;
      acc += (count[s] + 63) / 64 * 64;
    }
    off[S] = acc;
  }
}

// ------------------------------------------------------ fragment -> plain --
template <int TY>
__global__ void frag_to_plain_kernel(const TE<TY>* frag, int G, long gsi, int N, int Kd, int swf, int transpose,
                                     TE<TY>* out, long gso, long ldo) {
  const long total = (long)G * N * Kd;
  const int KS = Kd / 16;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const int g = (int)(i / ((long)N * Kd));
    const long rem = i - (long)g * N * Kd;
    const int n = (int)(rem / Kd), k = (int)(rem % Kd);
    const int ks = (k >> 6) * 4 + ((k & 31) >> 3), h = (k & 63) >> 5, e = k & 7;
    const long src = (((long)(n >> 5) * KS + ks) * 64 + (n & 31) + 32 * h) * 8 + e;
    int nl = n;
    if (swf > 0) nl = ((n >> 5) & 1) * swf + (n >> 6) * 32 + (n & 31);
    const long dst = transpose ? (long)k * ldo + nl : (long)nl * ldo + k;
    out[g * gso + dst] = frag[g * gsi + src];
  }
}

// ----------------------------------------------------- activation backward --
__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float gelu_t(float z, float& dgelu) {
  const float c = 0.7978845608028654f;
  const float u = c * (z + 0.044715f * z * z * z);
  const float t = tanhf(u);
  dgelu = 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * c * (1.0f + 3.0f * 0.044715f * z * z);
  return 0.5f * z * (1.0f + t);
}

// block-wide sum of NV values per thread (256 threads), result in red[0..NV)
template <int NV>
__device__ void block_sum(float (&v)[NV], float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float x = v[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    v[i] = x;
  }
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) red[wv * NV + i] = v[i];
  __syncthreads();
  if (tid < NV) red[4 * NV + tid] = red[tid] + red[NV + tid] + red[2 * NV + tid] + red[3 * NV + tid];
  __syncthreads();
}

// One workgroup per group row; the row's chosen experts one after another.
template <int TY>
__global__ void __launch_bounds__(256) act_bwd_kernel(ActBwdArgs a) {
  const int row = blockIdx.x;
  if (row >= a.R) return;
  __shared__ float red[5 * 49];
  const int ar = a.garow[row];
  const int t = ar / a.kg, rank = ar % a.kg;
  const int f = a.f, Pin = a.Pin, tid = threadIdx.x;
  const float* zb = a.Zb + (long)row * Pin * f;
  const float* dr = a.D + (long)row * f;
  float* dzb = a.dZbar + (long)row * Pin * f;
  float* hb = a.hbar + (long)row * f;
  for (int c = tid; c < f; c += 256) {
    hb[c] = 0.f;
    for (int p = 0; p < Pin; ++p) dzb[p * f + c] = 0.f;
  }
  for (int sl = 0; sl < a.ke; ++sl) {
    const int slot = rank * a.ke + sl;
    const long asg = (long)t * a.k + slot;
    const int i = a.idx[asg];
    const int j = i % a.K;
    const float wt = a.w[asg];
    float ug[16], uu[16], ev[16];
#pragma unroll
    for (int rho = 0; rho < 16; ++rho) {
      ug[rho] = a.r ? a.U[(long)row * a.NU + (j * Pin + 0) * 16 + rho] : 0.f;
      uu[rho] = (a.r && Pin > 1) ? a.U[(long)row * a.NU + (j * Pin + 1) * 16 + rho] : 0.f;
      ev[rho] = a.r ? a.Eb[(long)row * a.NE + j * 16 + rho] : 0.f;
    }
    // per-thread partial sums: q (dz B1, Pin x 16), u2 (h A2, 16), <D, h>
    float part[49];
#pragma unroll
    for (int x = 0; x < 49; ++x) part[x] = 0.f;
    const float* b1g = a.B1p + ((long)i * Pin + 0) * f * 16;
    const float* b1u = a.B1p + ((long)i * Pin + (Pin > 1 ? 1 : 0)) * f * 16;
    const float* ad = a.Adp + (long)i * f * 16;
    TE<TY>* dzo = static_cast<TE<TY>*>(a.dz) + asg * Pin * f;
    TE<TY>* who = static_cast<TE<TY>*>(a.wh) + asg * f;
    for (int c = tid; c < f; c += 256) {
      float zg = zb[c], zu = Pin > 1 ? zb[f + c] : 0.f;
      float dh = dr[c];
      if (a.r) {
#pragma unroll
        for (int rho = 0; rho < 16; ++rho) {
          zg += ug[rho] * b1g[c * 16 + rho];
          if (Pin > 1) zu += uu[rho] * b1u[c * 16 + rho];
          dh += ev[rho] * ad[c * 16 + rho];
        }
      }
      dh *= wt;
      float h, dzg, dzu = 0.f;
      if (a.act == ACT_SWIGLU) {
        const float sg = sigm(zg), sl_ = zg * sg;
        h = sl_ * zu;
        dzu = dh * sl_;
        dzg = dh * zu * sg * (1.0f + zg * (1.0f - sg));
      } else {
        float dg;
        h = gelu_t(zg, dg);
        dzg = dh * dg;
      }
      dzb[c] += dzg;
      if (Pin > 1) dzb[f + c] += dzu;
      hb[c] += wt * h;
      dzo[c] = from_f32<TY>(dzg);
      if (Pin > 1) dzo[f + c] = from_f32<TY>(dzu);
      who[c] = from_f32<TY>(wt * h);
      part[48] += dr[c] * h;
      if (a.r) {
#pragma unroll
        for (int rho = 0; rho < 16; ++rho) {
          part[rho] += dzg * b1g[c * 16 + rho];
          if (Pin > 1) part[16 + rho] += dzu * b1u[c * 16 + rho];
          part[32 + rho] += h * ad[c * 16 + rho];
        }
      }
    }
    block_sum<49>(part, red);
    if (tid < 16) {
      a.q[asg * Pin * 16 + tid] = red[4 * 49 + tid];
      if (Pin > 1) a.q[asg * Pin * 16 + 16 + tid] = red[4 * 49 + 16 + tid];
      a.wu2[asg * 16 + tid] = wt * red[4 * 49 + 32 + tid];
      a.ea[asg * 16 + tid] = ev[tid];
      a.ua[asg * Pin * 16 + tid] = ug[tid];
      if (Pin > 1) a.ua[asg * Pin * 16 + 16 + tid] = uu[tid];
    }
    if (tid == 0) {
      float dw = red[4 * 49 + 48];
      for (int rho = 0; rho < 16; ++rho) dw += ev[rho] * red[4 * 49 + 32 + rho];
      a.dw[asg] = dw;
    }
    __syncthreads();
  }
}

// --------------------------------------------------- token: router + dX ----
// One workgroup per token: softmax backward of the gate (w = p_g q_j), then
// dX = sum over the token's group rows of dXb + residual and router terms.
template <int XT>
__global__ void __launch_bounds__(256) tok_bwd_kernel(TokBwdArgs a) {
  const int t = blockIdx.x;
  if (t >= a.T) return;
  __shared__ float dsv[MAX_KG];
  __shared__ float dev[MAX_SLOTS];
  const int tid = threadIdx.x;
  if (tid == 0) {
    float pg[MAX_KG], dp[MAX_KG];
    float sp = 0.f;
    for (int g = 0; g < a.kg; ++g) {
      float p = 0.f, dpg = 0.f;
      for (int b = 0; b < a.ke; ++b) p += a.w[(long)t * a.k + g * a.ke + b];
      pg[g] = p;
      float qdq = 0.f;
      for (int b = 0; b < a.ke; ++b) {
        const long s = (long)t * a.k + g * a.ke + b;
        const float q = p > 0.f ? a.w[s] / p : 0.f;
        dpg += a.dw[s] * q;
        qdq += q * a.dw[s] * p;
      }
      dp[g] = dpg;
      sp += p * dpg;
      for (int b = 0; b < a.ke; ++b) {
        const long s = (long)t * a.k + g * a.ke + b;
        const float q = p > 0.f ? a.w[s] / p : 0.f;
        dev[g * a.ke + b] = a.K > 1 ? q * (a.dw[s] * p - qdq) : 0.f;
      }
    }
    for (int g = 0; g < a.kg; ++g) dsv[g] = pg[g] * (dp[g] - sp);
  }
  __syncthreads();
  // logit gradients out: ds [T][kg], de [T][kg][K] (zeros for the unchosen)
  for (int x = tid; x < a.kg * (1 + a.K); x += 256) {
    const int g = x / (1 + a.K), c = x % (1 + a.K);
    float v;
    if (c == 0) {
      v = dsv[g];
    } else {
      v = 0.f;
      for (int b = 0; b < a.ke; ++b) {
        const int ii = a.idx[(long)t * a.k + g * a.ke + b];
        if (ii % a.K == c - 1) v = dev[g * a.ke + b];
      }
    }
    a.ds[((long)t * a.kg + g) * (1 + a.K) + c] = v;
  }
  // dX
  for (int cc = tid; cc < a.d; cc += 256) {
    float v = 0.f;
    const float* wcol = a.Wr + ((long)(cc >> 4) * a.NCp) * 16 + (cc & 15);
    for (int g = 0; g < a.kg; ++g) {
      const int row = a.grow[(long)t * a.kg + g];
      v += a.dXb[(long)row * a.d + cc];
      const int gg = a.gidx[(long)t * a.kg + g];
      v += dsv[g] * wcol[gg * 16];
      for (int b = 0; b < a.ke; ++b) {
        const long s = (long)t * a.k + g * a.ke + b;
        const int ii = a.idx[s];
        if (a.K > 1) v += dev[g * a.ke + b] * wcol[(a.G + ii) * 16];
        if (a.r) {
          for (int p = 0; p < a.Pin; ++p) {
            const float* qv = a.q + (s * a.Pin + p) * 16;
            const float* at = a.Atp + (((long)ii * a.Pin + p) * a.d + cc) * 16;
#pragma unroll
            for (int rho = 0; rho < 16; ++rho) v += qv[rho] * at[rho];
          }
        }
      }
    }
    static_cast<TE<XT>*>(a.dX)[(long)t * a.d + cc] = from_f32<XT>(v);
  }
}

__global__ void invert_rows_kernel(const int* garow, int R, int* grow) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) grow[garow[r]] = r;
}

__global__ void assign_rows_kernel(const int* perm, const int* offsets, const int* idx, int E, int k, int Na,
                                   int* arow) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= Na) return;
  // expert of position p: the last e with offsets[e] <= p
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  const int t = perm[p];
  int slot = 0;
  for (int s = 0; s < k; ++s)
    if (idx[(long)t * k + s] == lo) slot = s;
  arow[p] = t * k + slot;
}

__global__ void seg_colsum_kernel(const float* in, long ld_in, int ncols, const int* start, const int* count,
                                  const int* in_map, float* out, long ld_out) {
  const int s = blockIdx.x;
  __shared__ float part[256];
  for (int c = 0; c < ncols; ++c) {
    float v = 0.f;
    for (int r = threadIdx.x; r < count[s]; r += 256) {
      const long pos = (long)start[s] + r;
      const long row = in_map ? in_map[pos] : pos;
      v += in[row * ld_in + c];
    }
    part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
      __syncthreads();
    }
    if (threadIdx.x == 0) out[(long)s * ld_out + c] = part[0];
    __syncthreads();
  }
}

template <int TY>
__global__ void stack_factors_kernel(const float* src, int G, int K, int P, int n, int rows_out, TE<TY>* out) {
  const long total = (long)G * rows_out * n;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const int g = (int)(i / ((long)rows_out * n));
    const long rem = i - (long)g * rows_out * n;
    const int row = (int)(rem / n), k = (int)(rem % n);
    const int j = row / (P * 16), p = (row / 16) % P, rho = row % 16;
    float v = 0.f;
    if (j < K) v = src[((((long)g * K + j) * P + p) * n + k) * 16 + rho];
    out[i] = from_f32<TY>(v);
  }
}

__global__ void zero_f_kernel(float* p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0.f;
}

}  // namespace

hipError_t launch_bgemm(int ty, const BGemmArgs& a, hipStream_t st) {
  const int NT = (a.N + BT - 1) / BT;
  long blocks;
  if (a.mode == 0) blocks = ((long)a.max_rows / BT + a.S) * NT;
  else blocks = (long)a.S * ((a.M + BT - 1) / BT) * NT;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(256);
#define BG(TY, SA) hipLaunchKernelGGL((bgemm_kernel<TY, SA>), grid, block, 0, st, a)
  if (ty == DT_F32) {
    BG(DT_F32, DT_F32);
  } else if (ty == DT_F16) {
    if (a.a_dtype == DT_F32) BG(DT_F16, DT_F32);
    else if (a.a_dtype == DT_BF16) BG(DT_F16, DT_BF16);
    else BG(DT_F16, DT_F16);
  } else {
    if (a.a_dtype == DT_F32) BG(DT_BF16, DT_F32);
    else BG(DT_BF16, DT_BF16);
  }
#undef BG
  return hipGetLastError();
}

hipError_t launch_gather_t(int ty, const TransArgs& a, hipStream_t st) {
  if (a.max_cols_k <= 0 || a.ncols <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.max_cols_k + 63) / 64), (unsigned)((a.ncols + 63) / 64)), block(256);
#define GT(TY, SI) hipLaunchKernelGGL((gather_t_kernel<TY, SI>), grid, block, 0, st, a)
  if (ty == DT_F32) {
    GT(DT_F32, DT_F32);
  } else if (ty == DT_F16) {
    if (a.in_dtype == DT_F32) GT(DT_F16, DT_F32);
    else if (a.in_dtype == DT_BF16) GT(DT_F16, DT_BF16);
    else GT(DT_F16, DT_F16);
  } else {
    if (a.in_dtype == DT_F32) GT(DT_BF16, DT_F32);
    else GT(DT_BF16, DT_BF16);
  }
#undef GT
  return hipGetLastError();
}

hipError_t launch_pad_scan(const int* count, int S, int* kpad_off, hipStream_t st) {
  hipLaunchKernelGGL(pad_scan_kernel, dim3(1), dim3(64), 0, st, count, S, kpad_off);
  return hipGetLastError();
}

hipError_t launch_frag_to_plain(int ty, const void* frag, int G, long gsi, int N, int Kd, int swf, bool transpose,
                                void* out, long gso, long ldo, hipStream_t st) {
  dim3 grid(2048), block(256);
  if (ty == DT_F32)
    hipLaunchKernelGGL(frag_to_plain_kernel<DT_F32>, grid, block, 0, st, static_cast<const float*>(frag), G, gsi, N,
                       Kd, swf, transpose ? 1 : 0, static_cast<float*>(out), gso, ldo);
  else
    hipLaunchKernelGGL(frag_to_plain_kernel<DT_F16>, grid, block, 0, st, static_cast<const uint16_t*>(frag), G, gsi,
                       N, Kd, swf, transpose ? 1 : 0, static_cast<uint16_t*>(out), gso, ldo);
  return hipGetLastError();
}

hipError_t launch_act_bwd(int ty, const ActBwdArgs& a, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  dim3 grid(a.R), block(256);
  switch (ty) {
    case DT_F32: hipLaunchKernelGGL(act_bwd_kernel<DT_F32>, grid, block, 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(act_bwd_kernel<DT_F16>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(act_bwd_kernel<DT_BF16>, grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_tok_bwd(const TokBwdArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  dim3 grid(a.T), block(256);
  switch (a.x_dtype) {
    case DT_F32: hipLaunchKernelGGL(tok_bwd_kernel<DT_F32>, grid, block, 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(tok_bwd_kernel<DT_F16>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(tok_bwd_kernel<DT_BF16>, grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_invert_rows(const int* garow, int R, int* grow, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(invert_rows_kernel, dim3((R + 255) / 256), dim3(256), 0, st, garow, R, grow);
  return hipGetLastError();
}

hipError_t launch_assign_rows(const int* perm, const int* offsets, const int* idx, int E, int k, int Na, int* arow,
                              hipStream_t st) {
  if (Na <= 0) return hipSuccess;
  hipLaunchKernelGGL(assign_rows_kernel, dim3((Na + 255) / 256), dim3(256), 0, st, perm, offsets, idx, E, k, Na, arow);
  return hipGetLastError();
}

hipError_t launch_seg_colsum(const float* in, long ld_in, int ncols, const int* start, const int* count,
                             const int* in_map, int S, float* out, long ld_out, hipStream_t st) {
  if (S <= 0 || ncols <= 0) return hipSuccess;
  hipLaunchKernelGGL(seg_colsum_kernel, dim3(S), dim3(256), 0, st, in, ld_in, ncols, start, count, in_map, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_stack_factors(int ty, const float* src, int G, int K, int P, int n, int rows_out, void* out,
                                hipStream_t st) {
  dim3 grid(1024), block(256);
  switch (ty) {
    case DT_F32: hipLaunchKernelGGL(stack_factors_kernel<DT_F32>, grid, block, 0, st, src, G, K, P, n, rows_out, static_cast<float*>(out)); break;
    case DT_F16: hipLaunchKernelGGL(stack_factors_kernel<DT_F16>, grid, block, 0, st, src, G, K, P, n, rows_out, static_cast<uint16_t*>(out)); break;
    default: hipLaunchKernelGGL(stack_factors_kernel<DT_BF16>, grid, block, 0, st, src, G, K, P, n, rows_out, static_cast<uint16_t*>(out)); break;
  }
  return hipGetLastError();
}

hipError_t launch_zero_f(float* p, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f_kernel, dim3(1024), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace cefn
