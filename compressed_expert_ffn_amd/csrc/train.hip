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
// gate.  The wide GEMMs run the forward pass's tile engine (rows through
// LDS, fragment-major column operands), over row segments (a group's rows,
// an expert's positions) or k segments (a group's rows, transposed); the
// thin factor gradients are sums over an expert's positions with the rows
// transposed in LDS; the activation step walks tiles of one expert's
// positions with that expert's factor rows in LDS; dX and the gate's
// softmax backward are assembled per token.
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

// Mode R: row tile i (of TR rows) of the segments, through the tile prefix
// (binary search) when there is one, else by walking the segments.
template <int TR>
__device__ __forceinline__ bool seg_tile(const BGemmArgs& a, int i, int& s, int& m0, int& M) {
  if (a.tile_off) {
    if (i >= a.tile_off[a.S]) return false;
    // the last segment whose first tile is <= i (never an empty one)
    int lo = 0, hi = a.S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_off[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    s = lo;
    m0 = (i - a.tile_off[lo]) * TR;
    M = a.seg_count[lo];
    return true;
  }
  for (int q = 0; q < a.S; ++q) {
    const int cnt = a.seg_count[q];
    const int mt = (cnt + TR - 1) / TR;
    if (i < mt) {
      s = q;
      m0 = i * TR;
      M = cnt;
      return true;
    }
    i -= mt;
  }
  return false;
}

template <int TY, int SA>
__global__ void __launch_bounds__(256) bgemm_kernel(BGemmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int NT = (a.N + BT - 1) / BT;
  int s = 0, m0 = 0, M = 0, K = 0, n0 = 0;
  long crow0 = 0, kofs = 0;
  if (a.mode == 0) {
    const int i = blockIdx.x;
    n0 = (i % NT) * BT;
    if (!seg_tile<BT>(a, i / NT, s, m0, M)) return;
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
  // B rows ride the lane index of the MFMA result and A rows its register
  // index, so a store writes 32 consecutive columns of one row of C.
  f16v acc[2][2];
  zero_acc<2, 2>(acc);
  const int KT = K / KB;
  if (KT > 0) {
    TDirect<TY, TY, 2> bt;
    const TE<TY>* bbase = static_cast<const TE<TY>*>(a.b) + (a.mode == 0 ? (long)s * a.b_sstride : kofs);
    bt.init(bbase, a.ldb, lane, [&](int t) -> long {
      const int n = n0 + wn * 64 + t * 32 + (lane & 31);
      return n < a.N ? n : -1;
    });
    BOperand<SA, TY> ao;
    const TE<SA>* abase = static_cast<const TE<SA>*>(a.a) + kofs;
    ao.td.init(abase, a.lda, lane, [&](int c) -> long {
      const int m = m0 + wm * 64 + c * 32 + (lane & 31);
      if (m >= M) return -1;
      if (a.mode == 1) return m;
      const long pos = crow0 + m;
      return a.a_map ? (long)(a.a_map[pos] / a.a_div) : pos;
    });
    Mainloop<TY, 2, 2, TDirect<TY, TY, 2>, BOperand<SA, TY>, 1> ml{bt, ao, lane};
    ml.template run<typename TDirect<TY, TY, 2>::Raw[2][4], typename BOperand<SA, TY>::Raw[2][4]>(KT, acc);
  }
  float* cbase = a.c + (a.mode == 0 ? crow0 * a.ldc : (long)s * a.c_sstride);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = n0 + wn * 64 + t * 32 + (lane & 31);
    if (n >= a.n_store) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + c * 32 + acc32_row(v, lane);
        if (m < M) cbase[(long)m * a.ldc + n] = acc[t][c][v];
      }
  }
}

// Index of element (n, k) in a fragment-major matrix of KS k-steps.
__device__ __forceinline__ long frag_index(long n, long k, long KS) {
  const long ks = (k >> 6) * 4 + ((k & 31) >> 3);
  return ((n >> 5) * KS + ks) * 512 + ((n & 31) + 32 * ((k & 63) >> 5)) * 8 + (k & 7);
}

// ------------------------------------------------------ wide segment GEMM --
// 32 RT rows of A (LDS, double-buffered) x 256 columns of B (four wavefronts
// of 64 columns, fragment-major, straight from memory): the forward pass's
// main loop with plain gathered rows on the token side.  KT = 0 (an empty
// k segment) stores zeros.
template <int TY, int SA, int RT>
__global__ void __launch_bounds__(256, (TY == DT_F32 || SA == DT_F32) ? 1 : 2) fgemm_kernel(BGemmArgs a) {
  using F = FragT<TY>;
  constexpr int FM = 32 * RT, FN = 256;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  F* tl = reinterpret_cast<F*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NT = (a.N + FN - 1) / FN;
  int s = 0, m0 = 0, M = 0, K = 0, n0 = 0;
  long crow0 = 0, kofs = 0;
  if (a.mode == 0) {
    const int i = blockIdx.x;
    n0 = (i % NT) * FN;
    if (!seg_tile<FM>(a, i / NT, s, m0, M)) return;
    K = a.K;
    crow0 = a.seg_start[s];
  } else {
    const int MT = (a.M + FM - 1) / FM;
    int i = blockIdx.x;
    n0 = (i % NT) * FN;
    i /= NT;
    m0 = (i % MT) * FM;
    s = i / MT;
    if (s >= a.S) return;
    M = a.M;
    kofs = a.kpad_off[s];
    K = a.kpad_off[s + 1] - a.kpad_off[s];
  }
  const int NB = (a.N + 63) / 64 * 2;  // 32-column blocks of B
  const int nbw = n0 / 32 + wave * 2;
  const bool active = nbw * 32 < a.N;
  const int nb0 = active ? nbw : NB - 2;
  f16v acc[RT][2];
  zero_acc<RT, 2>(acc);
  const int KT = K / KB;
  if (KT > 0) {
    TShared<SA, TY, RT> to;
    to.init(static_cast<const TE<SA>*>(a.a) + kofs, a.lda, [&](int blk, int r) -> long {
      const int m = m0 + blk * 32 + r;
      if (m >= M) return -1;
      if (a.mode == 1) return m;
      const long pos = crow0 + m;
      return a.a_map ? (long)(a.a_map[pos] / a.a_div) : pos;
    });
    const F* bb = static_cast<const F*>(a.b) + (a.mode == 0 ? (long)s * a.b_sstride / 8 : 0);
    WPlain<TY> ws{bb, (int)(a.mode == 0 ? K / 16 : a.ldb / 16)};
    ws.ks0 = (int)(kofs / 16);
    MainloopTW<TY, RT, 2, TShared<SA, TY, RT>, WPlain<TY>, 1> ml{to, ws, nb0, tl, lane};
    ml.run(KT, acc);
  }
  if (!active) return;
  float* cbase = a.c + (a.mode == 0 ? crow0 * a.ldc : (long)s * a.c_sstride);
  const bool vec = ((reinterpret_cast<uintptr_t>(a.c) | (uintptr_t)(a.ldc * 4) | (uintptr_t)(a.c_sstride * 4)) & 15) == 0;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int m = m0 + t * 32 + (lane & 31);
    if (m >= M) continue;
    float* crow = cbase + (long)m * a.ldc;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int nb = nb0 + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = acc32_row(4 * q, lane);  // 4 consecutive columns nl .. nl + 3
        const int n = nb * 32 + nl;
        const int col = a.swf > 0 ? ((nb & 1) * a.swf + (nb >> 1) * 32 + nl) : n;
        if (vec && n + 3 < a.n_store) {
          *reinterpret_cast<f4v*>(crow + col) = f4v{acc[t][c][4 * q], acc[t][c][4 * q + 1], acc[t][c][4 * q + 2],
                                                     acc[t][c][4 * q + 3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n + i < a.n_store) crow[col + i] = acc[t][c][4 * q + i];
        }
      }
    }
  }
}

template <int TY>
__global__ void plain_to_frag_kernel(const TE<TY>* in, int G, long gsi, int N, int Kd, TE<TY>* out, long gso) {
  const int Np = (N + 63) / 64 * 64;
  const long total = (long)G * Np * Kd;
  const long KS = Kd / 16;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const int g = (int)(i / ((long)Np * Kd));
    const long rem = i - (long)g * Np * Kd;
    const int n = (int)(rem / Kd), k = (int)(rem % Kd);
    out[g * gso + frag_index(n, k, KS)] = n < N ? in[g * gsi + (long)n * Kd + k] : from_f32<TY>(0.f);
  }
}

// ------------------------------------------------ thin transposed GEMM ----
// A workgroup owns 128 columns m of A for one segment and walks the
// segment's rows in chunks of 64: the chunk's A rows (128 contiguous values
// each) and B rows go to LDS transposed (k = row contiguous), then wavefront
// w takes m-block w: four 32x32x16 MFMA steps against the 32 B columns.
template <int TY, int SA>
__global__ void __launch_bounds__(256) tgemm_kernel(TGemmArgs a) {
  using F = FragT<TY>;
  constexpr int KP = 64 + (TY == DT_F32 ? 4 : 8);  // LDS row stride (16-byte rows of fragments)
  __shared__ __attribute__((aligned(16))) TE<TY> lA[128 * KP];
  __shared__ __attribute__((aligned(16))) TE<TY> lB[32 * KP];
  const int s = blockIdx.y, m0 = blockIdx.x * 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int start = a.seg_start[s], cnt = a.seg_count[s];
  const TE<SA>* A = static_cast<const TE<SA>*>(a.a);
  f16v acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int pr = tid >> 2, q4 = tid & 3;  // loader: row pr of the chunk, quarter q4
  for (int c0 = 0; c0 < cnt; c0 += 64) {
    const bool ok = c0 + pr < cnt;
    long row = 0;
    if (ok) {
      const long p = (long)start + c0 + pr;
      row = a.a_map ? (long)(a.a_map[p] / a.a_div) : p;
    }
    __syncthreads();  // the previous chunk's fragments are read
    // A: 32 values m = q4 * 32 .. + 31 of row pr
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = q4 * 32 + j * 8;
      float v[8];
      if (ok && m0 + m < a.M) {
        const RawT<SA> raw = ld_raw<SA>(A + row * a.lda + a.a_c0 + m0 + m);
        if constexpr (SA == DT_F32) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = raw[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t h = static_cast<uint16_t>((raw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            v[e] = SA == DT_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lA[(m + e) * KP + pr] = from_f32<TY>(v[e]);
    }
    // B: 8 values n = q4 * 8 .. + 7 of row pr
    {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = q4 * 8 + e;
        v[e] = (ok && n < a.N) ? a.b[((long)start + c0 + pr) * a.ldb + a.b_c0 + n] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lB[(q4 * 8 + e) * KP + pr] = from_f32<TY>(v[e]);
    }
    __syncthreads();
    const TE<TY>* ar = lA + (wave * 32 + (lane & 31)) * KP + 8 * (lane >> 5);
    const TE<TY>* br = lB + (lane & 31) * KP + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      F fa, fb;
      if constexpr (TY == DT_F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          fa[e] = ar[ks * 16 + e];
          fb[e] = br[ks * 16 + e];
        }
      } else {
        fa = *reinterpret_cast<const F*>(ar + ks * 16);
        fb = *reinterpret_cast<const F*>(br + ks * 16);
      }
      acc = mfma32<TY>(fa, fb, acc);
    }
  }
  const int n = lane & 31;
  if (n >= a.N || (n & 15) >= a.n_store) return;
  float* cb = (n < 16 ? a.c_lo : a.c_hi) + (long)s * a.c_sstride + (n & 15);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = m0 + wave * 32 + acc32_row(v, lane);
    if (m < a.M) cb[(long)m * a.ldc] = acc[v];
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
  const TE<SI>* in = static_cast<const TE<SI>*>(a.in);
  // rows of 8 consecutive columns per thread when the source allows it
  const bool vin = (a.ld_in % 8 == 0) && (a.c0 % 8 == 0) && (a.ncols % 8 == 0);
  if (vin) {
    for (int i = tid; i < 64 * 8; i += 256) {
      const int rr = i >> 3, cq = (i & 7) * 8;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (r0 + rr < cnt && c0 + cq < a.ncols) {
        const long pos = (long)a.start[s] + r0 + rr;
        const long row = a.in_map ? (long)(a.in_map[pos] / a.in_div) : pos;
        const RawT<SI> raw = ld_raw<SI>(in + row * a.ld_in + a.c0 + c0 + cq);
        if constexpr (SI == DT_F32) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = raw[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t h = static_cast<uint16_t>((raw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            v[e] = SI == DT_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tileS[rr][cq + e] = v[e];
    }
  } else {
    for (int i = tid; i < 64 * 64; i += 256) {
      const int rr = i / 64, cc = i % 64;  // source row r0 + rr, column c0 + cc
      float v = 0.f;
      if (r0 + rr < cnt && c0 + cc < a.ncols) {
        const long pos = (long)a.start[s] + r0 + rr;
        const long row = a.in_map ? (long)(a.in_map[pos] / a.in_div) : pos;
        v = load_as_f32<SI>(in, row * a.ld_in + a.c0 + c0 + cc);
      }
      tileS[rr][cc] = v;
    }
  }
  __syncthreads();
  // 8 consecutive k of one output row per thread (one 16- or 32-byte store)
  TE<TY>* out = static_cast<TE<TY>*>(a.out);
  const int rows = a.frag ? (a.ncols + 31) / 32 * 32 : a.ncols;
  for (int i = tid; i < 64 * 8; i += 256) {
    const int cc = i >> 3, rq = (i & 7) * 8;
    if (c0 + cc >= rows) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tileS[rq + e][cc];
    TE<TY>* dst = out + (a.frag ? frag_index(c0 + cc, kc + rq, a.ld_out / 16) : (long)(c0 + cc) * a.ld_out + kc + rq);
    if constexpr (TY == DT_F32) {
      reinterpret_cast<f4v*>(dst)[0] = f4v{v[0], v[1], v[2], v[3]};
      reinterpret_cast<f4v*>(dst)[1] = f4v{v[4], v[5], v[6], v[7]};
    } else {
      u4v w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = static_cast<uint32_t>(from_f32<TY>(v[2 * q])) | (static_cast<uint32_t>(from_f32<TY>(v[2 * q + 1])) << 16);
      *reinterpret_cast<u4v*>(dst) = w;
    }
  }
}

// Exclusive prefix of ceil(count[s] / rows) * mult over S <= 1024 segments,
// by one workgroup of 1024 threads (off[S] = the total).
__global__ void __launch_bounds__(1024) seg_scan_kernel(const int* count, int S, int rows, int mult, int* off) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int v = tid < S ? (count[tid] + rows - 1) / rows * mult : 0;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wv; ++w) base += wsum[w];
  if (tid < S) off[tid] = base + inc - v;
  if (tid == S - 1) off[S] = base + inc;
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

// Four consecutive values of type TY, as one 8- or 16-byte access.
template <int TY>
__device__ __forceinline__ void store4(TE<TY>* p, const float (&v)[4]) {
  if constexpr (TY == DT_F32) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 u;
    u.x = (uint32_t)from_f32<TY>(v[0]) | ((uint32_t)from_f32<TY>(v[1]) << 16);
    u.y = (uint32_t)from_f32<TY>(v[2]) | ((uint32_t)from_f32<TY>(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
}
template <int TY>
__device__ __forceinline__ void load4_add(const TE<TY>* p, float (&v)[4]) {
  if constexpr (TY == DT_F32) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] += x.x; v[1] += x.y; v[2] += x.z; v[3] += x.w;
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const uint16_t h[4] = {(uint16_t)(u.x & 0xFFFFu), (uint16_t)(u.x >> 16), (uint16_t)(u.y & 0xFFFFu),
                           (uint16_t)(u.y >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += load_as_f32<TY>(h, i);
  }
}

// Per expert-list position (one wavefront each): assignment, row, weight
// and the u / e vectors.
__global__ void __launch_bounds__(256) gather_assign_kernel(AssignArgs a) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6), x = threadIdx.x & 63;
  if (p >= a.Na) return;
  // expert of position p: the last e with offsets[e] <= p
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.offsets[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  const int t = a.perm[p];
  // slot of expert lo among the token's k choices (lanes compare in parallel)
  const bool hit = x < a.k && a.idx[(long)t * a.k + x] == lo;
  const unsigned long long m = __ballot(hit);
  const int slot = m ? __ffsll((long long)m) - 1 : 0;
  const long asg = (long)t * a.k + slot;
  const int row = a.grow[(long)t * (a.k / a.ke) + slot / a.ke];
  if (x == 0) {
    a.arow[p] = (int)asg;
    a.apos[asg] = p;
    a.prow[p] = row;
    a.pw[p] = a.w[asg];
  }
  if (a.r > 0) {
    const int j = lo % a.K;
    a.ua[(long)p * 64 + x] = x < a.Pin * 16 ? a.U[(long)row * a.NU + (long)j * a.Pin * 16 + x] : 0.f;
    if (x < 16) a.ea[(long)p * 16 + x] = a.Eb[(long)row * a.NE + j * 16 + x];
  }
}

// A workgroup takes 64 positions of one expert (4 lanes per position, each
// lane 4 consecutive columns of every 16) over its split's 64-column chunks;
// the chunk's factor rows B1_gate, B1_up, A2 [64][16] sit in LDS, so each is
// read from memory once per tile instead of once per assignment.  The
// column sums stay in registers and are reduced over the 4 lanes at the end.
template <int TY, int PIN, bool RES>
__global__ void __launch_bounds__(256) act_kernel(ActArgs a) {
  __shared__ float4 fs[3][64][4];
  const int tile = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  if (tile * 64 >= a.kpad[a.E]) return;
  // expert of the tile: the last e with kpad[e] <= tile * 64 (never empty)
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.kpad[mid] <= tile * 64) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int p0 = a.offsets[e] + (tile * 64 - a.kpad[e]);
  const int n = min(64, a.offsets[e] + a.counts[e] - p0);
  const int pl = tid >> 2, cg = tid & 3;
  const bool valid = pl < n;
  const int p = valid ? p0 + pl : p0;
  const int f = a.f;
  const int row = a.prow[p];
  const float wt = valid ? a.pw[p] : 0.f;
  float ug[16], uu[16], ev[16];
  float qg[16], qu[16], u2[16], dd = 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    ug[x] = RES ? a.ua[(long)p * 64 + x] : 0.f;
    uu[x] = (RES && PIN > 1) ? a.ua[(long)p * 64 + 16 + x] : 0.f;
    ev[x] = RES ? a.ea[(long)p * 16 + x] : 0.f;
    qg[x] = qu[x] = u2[x] = 0.f;
  }
  const int nch = f / 64;
  const int ch0 = (int)((long)split * nch / a.NS), ch1 = (int)((long)(split + 1) * nch / a.NS);
  const float* zrow = a.Zb + (long)row * PIN * f;
  const float* drow = a.D + (long)row * f;
  TE<TY>* dzo = static_cast<TE<TY>*>(a.dz) + (long)p * PIN * f;
  TE<TY>* who = static_cast<TE<TY>*>(a.wh) + (long)p * f;
  const float4* b1g = reinterpret_cast<const float4*>(a.B1p + (long)e * PIN * f * 16);
  const float4* b1u = reinterpret_cast<const float4*>(a.B1p + ((long)e * PIN + (PIN - 1)) * f * 16);
  const float4* adp = reinterpret_cast<const float4*>(a.Adp + (long)e * f * 16);
  for (int ch = ch0; ch < ch1; ++ch) {
    const int c0 = ch * 64;
    if (RES) {
      __syncthreads();
      fs[0][tid >> 2][tid & 3] = b1g[(long)c0 * 4 + tid];
      if (PIN > 1) fs[1][tid >> 2][tid & 3] = b1u[(long)c0 * 4 + tid];
      fs[2][tid >> 2][tid & 3] = adp[(long)c0 * 4 + tid];
      __syncthreads();
    }
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
      const int cl = cg * 4 + 16 * i, c = c0 + cl;
      const float4 zg4 = *reinterpret_cast<const float4*>(zrow + c);
      float4 zu4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (PIN > 1) zu4 = *reinterpret_cast<const float4*>(zrow + f + c);
      const float4 d4 = *reinterpret_cast<const float4*>(drow + c);
      const float zgv[4] = {zg4.x, zg4.y, zg4.z, zg4.w}, zuv[4] = {zu4.x, zu4.y, zu4.z, zu4.w};
      const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
      float og[4], ou[4], oh[4];
      // one column at a time (keeps the factor values of a single column live)
#pragma unroll 1
      for (int jj = 0; jj < 4; ++jj) {
        float bg[16], bu[16], ba[16];
        float zg = 0.f, zu = 0.f, dh = 0.f, dj = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (x == jj) {
            zg = zgv[x];
            zu = zuv[x];
            dj = dv[x];
          }
        dh = dj;
        if (RES) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 x = fs[0][cl + jj][q];
            bg[4 * q] = x.x; bg[4 * q + 1] = x.y; bg[4 * q + 2] = x.z; bg[4 * q + 3] = x.w;
            const float4 y = fs[2][cl + jj][q];
            ba[4 * q] = y.x; ba[4 * q + 1] = y.y; ba[4 * q + 2] = y.z; ba[4 * q + 3] = y.w;
            if (PIN > 1) {
              const float4 z = fs[1][cl + jj][q];
              bu[4 * q] = z.x; bu[4 * q + 1] = z.y; bu[4 * q + 2] = z.z; bu[4 * q + 3] = z.w;
            }
          }
#pragma unroll
          for (int rho = 0; rho < 16; ++rho) {
            zg += ug[rho] * bg[rho];
            if (PIN > 1) zu += uu[rho] * bu[rho];
            dh += ev[rho] * ba[rho];
          }
        }
        dh *= wt;
        float h, dzg, dzu = 0.f;
        if (a.act == ACT_SWIGLU) {
          const float sg = sigm(zg), sl = zg * sg;
          h = sl * zu;
          dzu = dh * sl;
          dzg = dh * zu * sg * (1.0f + zg * (1.0f - sg));
        } else {
          float dg;
          h = gelu_t(zg, dg);
          dzg = dh * dg;
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (x == jj) {
            og[x] = dzg;
            ou[x] = dzu;
            oh[x] = wt * h;
          }
        dd += dj * h;
        if (RES) {
#pragma unroll
          for (int rho = 0; rho < 16; ++rho) {
            qg[rho] += dzg * bg[rho];
            if (PIN > 1) qu[rho] += dzu * bu[rho];
            u2[rho] += h * ba[rho];
          }
        }
      }
      if (valid) {
        store4<TY>(dzo + c, og);
        if (PIN > 1) store4<TY>(dzo + f + c, ou);
        store4<TY>(who + c, oh);
      }
    }
  }
  // reduce over the 4 lanes of the position (adjacent lanes)
  dd += __shfl_xor(dd, 1);
  dd += __shfl_xor(dd, 2);
  if (RES) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      qg[x] += __shfl_xor(qg[x], 1);
      qg[x] += __shfl_xor(qg[x], 2);
      if (PIN > 1) {
        qu[x] += __shfl_xor(qu[x], 1);
        qu[x] += __shfl_xor(qu[x], 2);
      }
      u2[x] += __shfl_xor(u2[x], 1);
      u2[x] += __shfl_xor(u2[x], 2);
    }
  }
  if (valid && cg == 0) {
    float* po = a.part + ((long)split * a.Na + p) * ACT_PART;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      po[x] = qg[x];
      po[16 + x] = qu[x];
      po[32 + x] = u2[x];
    }
    po[48] = dd;
  }
}

// Activation backward on MFMAs (16-bit MFMA types, residual layers).  The
// tile's 64 positions x 64-column chunk is four 32 x 32 blocks, one per
// wavefront (position block pb = wave & 1, column block cb = wave >> 1),
// held like the forward pass's accumulators: lane = position, 16 columns
// per lane.  z_gate = Z + B1_gate u_gate is one 32x32x16 MFMA with Z as the
// accumulator (z_up and D + A2 e likewise); the column sums dz_gate B1_gate,
// dz_up B1_up and h A2 are MFMAs over the block's 32 columns with dz and h
// straight from registers (their k order is the columns a lane holds) and
// the factor rows read from LDS in that same order.  The two column-block
// wavefronts of a position block meet in LDS (fixed order) at the end.
template <int TY, int PIN>
__global__ void __launch_bounds__(256) act_mfma_kernel(ActArgs a) {
  using F = FragT<TY>;
  __shared__ float4 fs[3][64][4];
  __shared__ float xs[2][32][49];
  const int tile = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  if (tile * 64 >= a.kpad[a.E]) return;
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.kpad[mid] <= tile * 64) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int p0 = a.offsets[e] + (tile * 64 - a.kpad[e]);
  const int n = min(64, a.offsets[e] + a.counts[e] - p0);
  const int wave = tid >> 6, lane = tid & 63, pb = wave & 1, cb = wave >> 1, hh = lane >> 5;
  const int pl = pb * 32 + (lane & 31);
  const bool valid = pl < n;
  const int p = valid ? p0 + pl : p0;
  const int f = a.f, row = a.prow[p];
  const float wt = valid ? a.pw[p] : 0.f;
  float tmp[8];
  // second operands of the expansions (k = rank index 8 hh .. 8 hh + 7)
#pragma unroll
  for (int i = 0; i < 8; ++i) tmp[i] = a.ua[(long)p * 64 + 8 * hh + i];
  const F fug = to_frag<TY>(tmp);
#pragma unroll
  for (int i = 0; i < 8; ++i) tmp[i] = PIN > 1 ? a.ua[(long)p * 64 + 16 + 8 * hh + i] : 0.f;
  const F fuu = to_frag<TY>(tmp);
#pragma unroll
  for (int i = 0; i < 8; ++i) tmp[i] = a.ea[(long)p * 16 + 8 * hh + i];
  const F fe = to_frag<TY>(tmp);
  f16v qg, qu, u2;
#pragma unroll
  for (int v = 0; v < 16; ++v) qg[v] = qu[v] = u2[v] = 0.f;
  float dd = 0.f;
  const int nch = f / 64;
  const int ch0 = (int)((long)split * nch / a.NS), ch1 = (int)((long)(split + 1) * nch / a.NS);
  const float4* b1g = reinterpret_cast<const float4*>(a.B1p + (long)e * PIN * f * 16);
  const float4* b1u = reinterpret_cast<const float4*>(a.B1p + ((long)e * PIN + (PIN - 1)) * f * 16);
  const float4* adp = reinterpret_cast<const float4*>(a.Adp + (long)e * f * 16);
  TE<TY>* dzo = static_cast<TE<TY>*>(a.dz) + (long)p * PIN * f;
  TE<TY>* who = static_cast<TE<TY>*>(a.wh) + (long)p * f;
  const int cc = cb * 32, rho = lane & 31;
  for (int ch = ch0; ch < ch1; ++ch) {
    const int c0 = ch * 64;
    __syncthreads();
    fs[0][tid >> 2][tid & 3] = b1g[(long)c0 * 4 + tid];
    if (PIN > 1) fs[1][tid >> 2][tid & 3] = b1u[(long)c0 * 4 + tid];
    fs[2][tid >> 2][tid & 3] = adp[(long)c0 * 4 + tid];
    __syncthreads();
    // first operands of the expansions: row = column cc + lane % 32
    auto rowfrag = [&](int which) {
      const float4 x0 = fs[which][cc + (lane & 31)][2 * hh], x1 = fs[which][cc + (lane & 31)][2 * hh + 1];
      const float v8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      return to_frag<TY>(v8);
    };
    const F fbg = rowfrag(0);
    const F fad = rowfrag(2);
    // accumulators: element v is column cc + 8 (v / 4) + 4 hh + v % 4
    f16v zg, zu, dh;
    float dv[16];
    const float* zr = a.Zb + (long)row * PIN * f + c0 + cc + 4 * hh;
    const float* dr = a.D + (long)row * f + c0 + cc + 4 * hh;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 z4 = *reinterpret_cast<const float4*>(zr + 8 * q);
      const float4 d4 = *reinterpret_cast<const float4*>(dr + 8 * q);
      zg[4 * q] = z4.x; zg[4 * q + 1] = z4.y; zg[4 * q + 2] = z4.z; zg[4 * q + 3] = z4.w;
      dv[4 * q] = d4.x; dv[4 * q + 1] = d4.y; dv[4 * q + 2] = d4.z; dv[4 * q + 3] = d4.w;
      dh[4 * q] = d4.x; dh[4 * q + 1] = d4.y; dh[4 * q + 2] = d4.z; dh[4 * q + 3] = d4.w;
      if (PIN > 1) {
        const float4 u4 = *reinterpret_cast<const float4*>(zr + f + 8 * q);
        zu[4 * q] = u4.x; zu[4 * q + 1] = u4.y; zu[4 * q + 2] = u4.z; zu[4 * q + 3] = u4.w;
      } else {
        zu[4 * q] = zu[4 * q + 1] = zu[4 * q + 2] = zu[4 * q + 3] = 0.f;
      }
    }
    zg = mfma32<TY>(fbg, fug, zg);
    if (PIN > 1) zu = mfma32<TY>(rowfrag(1), fuu, zu);
    dh = mfma32<TY>(fad, fe, dh);
    float og[16], ou[16], oh[16], hv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float dhv = wt * dh[v];
      float h, dzg, dzu = 0.f;
      if (a.act == ACT_SWIGLU) {
        const float sg = sigm(zg[v]), sl = zg[v] * sg;
        h = sl * zu[v];
        dzu = dhv * sl;
        dzg = dhv * zu[v] * sg * (1.0f + zg[v] * (1.0f - sg));
      } else {
        float dgl;
        h = gelu_t(zg[v], dgl);
        dzg = dhv * dgl;
      }
      og[v] = dzg;
      ou[v] = dzu;
      oh[v] = wt * h;
      hv[v] = h;
      dd += dv[v] * h;
    }
    if (valid) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = c0 + cc + 8 * q + 4 * hh;
        const float g4[4] = {og[4 * q], og[4 * q + 1], og[4 * q + 2], og[4 * q + 3]};
        store4<TY>(dzo + col, g4);
        if (PIN > 1) {
          const float u4[4] = {ou[4 * q], ou[4 * q + 1], ou[4 * q + 2], ou[4 * q + 3]};
          store4<TY>(dzo + f + col, u4);
        }
        const float h4[4] = {oh[4 * q], oh[4 * q + 1], oh[4 * q + 2], oh[4 * q + 3]};
        store4<TY>(who + col, h4);
      }
    }
    // column sums: k-step s takes v = 8 s .. 8 s + 7, i.e. the columns
    // cc + 16 s + 8 (i / 4) + 4 hh + i % 4; factor rows rho < 16 (zero past)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float tg[8], tu[8], ta[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = cc + 16 * s + 8 * (i >> 2) + 4 * hh + (i & 3);
        tg[i] = rho < 16 ? reinterpret_cast<const float*>(&fs[0][col][0])[rho] : 0.f;
        tu[i] = (PIN > 1 && rho < 16) ? reinterpret_cast<const float*>(&fs[1][col][0])[rho] : 0.f;
        ta[i] = rho < 16 ? reinterpret_cast<const float*>(&fs[2][col][0])[rho] : 0.f;
      }
      qg = mfma32<TY>(to_frag<TY>(tg), to_frag<TY>(og + 8 * s), qg);
      if (PIN > 1) qu = mfma32<TY>(to_frag<TY>(tu), to_frag<TY>(ou + 8 * s), qu);
      u2 = mfma32<TY>(to_frag<TY>(ta), to_frag<TY>(hv + 8 * s), u2);
    }
  }
  // <D, h>: the two lane halves hold the block's two column halves
  dd += __shfl_xor(dd, 32);
  // lane (position lane % 32) holds rank index acc32_row(v, lane) for v < 8;
  // column block 1 hands its sums to column block 0
  __syncthreads();
  if (cb == 1) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int r = acc32_row(v, lane);
      xs[pb][lane & 31][r] = qg[v];
      xs[pb][lane & 31][16 + r] = qu[v];
      xs[pb][lane & 31][32 + r] = u2[v];
    }
    if (hh == 0) xs[pb][lane & 31][48] = dd;
  }
  __syncthreads();
  if (cb == 0 && valid) {
    float* po = a.part + ((long)split * a.Na + p) * ACT_PART;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int r = acc32_row(v, lane);
      po[r] = qg[v] + xs[pb][lane & 31][r];
      po[16 + r] = qu[v] + xs[pb][lane & 31][16 + r];
      po[32 + r] = u2[v] + xs[pb][lane & 31][32 + r];
    }
    if (hh == 0) po[48] = dd + xs[pb][lane & 31][48];
  }
}

// Without residuals: one wavefront per position, lanes along the columns
// (4 consecutive per lane, 256 per step), so every access is a contiguous
// run of the row; <D, h> is summed per lane in column order, then over the
// lanes, and written as the gate-weight gradient.
template <int TY, int PIN>
__global__ void __launch_bounds__(256) act_plain_kernel(ActArgs a, const int* arow, float* dw) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (p >= a.Na) return;
  const int f = a.f, row = a.prow[p];
  const float wt = a.pw[p];
  const float* zrow = a.Zb + (long)row * PIN * f;
  const float* drow = a.D + (long)row * f;
  TE<TY>* dzo = static_cast<TE<TY>*>(a.dz) + (long)p * PIN * f;
  TE<TY>* who = static_cast<TE<TY>*>(a.wh) + (long)p * f;
  float dd = 0.f;
  for (int c = lane * 4; c < f; c += 256) {
    const float4 zg4 = *reinterpret_cast<const float4*>(zrow + c);
    float4 zu4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (PIN > 1) zu4 = *reinterpret_cast<const float4*>(zrow + f + c);
    const float4 d4 = *reinterpret_cast<const float4*>(drow + c);
    const float zgv[4] = {zg4.x, zg4.y, zg4.z, zg4.w}, zuv[4] = {zu4.x, zu4.y, zu4.z, zu4.w};
    const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
    float og[4], ou[4], oh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float zg = zgv[j], zu = zuv[j], dh = wt * dv[j];
      float h, dzg, dzu = 0.f;
      if (a.act == ACT_SWIGLU) {
        const float sg = sigm(zg), sl = zg * sg;
        h = sl * zu;
        dzu = dh * sl;
        dzg = dh * zu * sg * (1.0f + zg * (1.0f - sg));
      } else {
        float dg;
        h = gelu_t(zg, dg);
        dzg = dh * dg;
      }
      og[j] = dzg;
      ou[j] = dzu;
      oh[j] = wt * h;
      dd += dv[j] * h;
    }
    store4<TY>(dzo + c, og);
    if (PIN > 1) store4<TY>(dzo + f + c, ou);
    store4<TY>(who + c, oh);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) dd += __shfl_xor(dd, o);
  if (lane == 0) dw[arow[p]] = dd;
}

// One wavefront per position: lane x < 49 sums value x over the splits.
__global__ void __launch_bounds__(256) act_finish_kernel(const float* part, int NS, int Na, int Pin, int r,
                                                         const float* pw, const float* ea, const int* arow, float* q,
                                                         float* wu2, float* dw) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6), x = threadIdx.x & 63;
  if (p >= Na) return;
  float acc = 0.f;
  if (x < 49)
    for (int s = 0; s < NS; ++s) acc += part[((long)s * Na + p) * ACT_PART + x];
  // <e, h A2> over lanes 32..47, added to <D, h> of lane 48 in a fixed order
  float t = (r > 0 && x >= 32 && x < 48) ? ea[(long)p * 16 + (x - 32)] * acc : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
  const float dd = __shfl(acc, 48);
  if (r > 0) {
    if (x < 32) q[(long)p * 64 + x] = (x < 16 || Pin > 1) ? acc : 0.f;
    else q[(long)p * 64 + x] = 0.f;
    if (x >= 32 && x < 48) wu2[(long)p * 16 + (x - 32)] = pw[p] * acc;
  }
  if (x == 0) dw[arow[p]] = dd + t;
}

// One workgroup per group row: dZbar and hbar as sums over its assignments.
template <int TY>
__global__ void __launch_bounds__(256) row_sums_kernel(const TE<TY>* dz, const TE<TY>* wh, const int* garow,
                                                       const int* apos, int kg, int ke, int k, int f, int Pin,
                                                       TE<TY>* dZbar, TE<TY>* hbar) {
  const int row = blockIdx.x;
  const int ar = garow[row];
  const int t = ar / kg, rank = ar % kg;
  int pos[MAX_SLOTS];
  for (int sl = 0; sl < ke; ++sl) pos[sl] = apos[(long)t * k + rank * ke + sl];
  const long W = (long)Pin * f;
  for (int c = threadIdx.x * 4; c < W; c += 1024) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < ke; ++sl) load4_add<TY>(dz + pos[sl] * W + c, v);
    store4<TY>(dZbar + row * W + c, v);
  }
  for (int c = threadIdx.x * 4; c < f; c += 1024) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < ke; ++sl) load4_add<TY>(wh + (long)pos[sl] * f + c, v);
    store4<TY>(hbar + (long)row * f + c, v);
  }
}

// --------------------------------------------------- token: router + dX ----
// One workgroup per (token, block of a.cols columns): softmax backward of
// the gate (w = p_g q_j; every column block of the token repeats it, the
// first one stores the logit gradients), then dX = sum over the token's
// group rows of dXb, over its assignments of dXr, plus the router terms.
template <int XT>
__global__ void __launch_bounds__(256) tok_kernel(TokArgs a) {
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
  // logit gradients out: ds [T][kg][1 + K] (zeros for the unchosen experts)
  for (int x = tid; blockIdx.y == 0 && x < a.kg * (1 + a.K); x += 256) {
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
  // this workgroup's columns of dX, 4 consecutive per thread
  __shared__ int srow[MAX_KG], sgg[MAX_KG], sex[MAX_SLOTS], spos[MAX_SLOTS];
  if (tid < a.kg) {
    srow[tid] = a.grow[(long)t * a.kg + tid];
    sgg[tid] = a.gidx[(long)t * a.kg + tid];
  }
  if (tid < a.k) {
    sex[tid] = a.idx[(long)t * a.k + tid];
    spos[tid] = a.r ? a.apos[(long)t * a.k + tid] : 0;
  }
  __syncthreads();
  const int cbeg = blockIdx.y * a.cols, cend = min(a.d, cbeg + a.cols);
  auto ld4 = [](const float* p) { return *reinterpret_cast<const float4*>(p); };
  for (int cc = cbeg + tid * 4; cc < cend; cc += 1024) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](float s, const float4& x) {
      v.x += s * x.x;
      v.y += s * x.y;
      v.z += s * x.z;
      v.w += s * x.w;
    };
    const float* wcol = a.Wr + ((long)(cc >> 4) * a.NCp) * 16 + (cc & 15);
    for (int g = 0; g < a.kg; ++g) {
      add(1.f, ld4(a.dXb + (long)srow[g] * a.d + cc));
      add(dsv[g], ld4(wcol + sgg[g] * 16));
      for (int b = 0; b < a.ke; ++b) {
        const int sl = g * a.ke + b;
        if (a.K > 1) add(dev[sl], ld4(wcol + (a.G + sex[sl]) * 16));
        if (a.r) add(1.f, ld4(a.dXr + (long)spos[sl] * a.d + cc));
      }
    }
    const float o[4] = {v.x, v.y, v.z, v.w};
    store4<XT>(static_cast<TE<XT>*>(a.dX) + (long)t * a.d + cc, o);
  }
}

__global__ void invert_rows_kernel(const int* garow, int R, int* grow) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) grow[garow[r]] = r;
}

template <int TY>
__global__ void a1t_kernel(const float* Atp, int E, int Pin, int d, TE<TY>* out) {
  const long total = (long)E * d * 64;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const int kk = (int)(i & 63);
    const long en = i >> 6;
    const int e = (int)(en / d), nn = (int)(en % d);
    float v = 0.f;
    if (kk < Pin * 16) v = Atp[(((long)e * Pin + kk / 16) * d + nn) * 16 + (kk & 15)];
    out[i] = from_f32<TY>(v);
  }
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

hipError_t launch_fgemm(int ty, const BGemmArgs& a, hipStream_t st) {
  if (a.N % 64) return hipErrorInvalidValue;
  const int RT = ty == DT_F32 ? 2 : 4, FM = 32 * RT;
  const int NT = (a.N + 255) / 256;
  long blocks;
  if (a.mode == 0) blocks = ((long)a.max_rows / FM + a.S) * NT;
  else blocks = (long)a.S * ((a.M + FM - 1) / FM) * NT;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(256);
  const size_t lds = (size_t)2 * RT * 4 * 64 * (ty == DT_F32 ? 32 : 16);
#define FG(TY, SA, R) hipLaunchKernelGGL((fgemm_kernel<TY, SA, R>), grid, block, lds, st, a)
  if (ty == DT_F32) {
    FG(DT_F32, DT_F32, 2);
  } else if (ty == DT_F16) {
    if (a.a_dtype == DT_F32) FG(DT_F16, DT_F32, 4);
    else if (a.a_dtype == DT_BF16) FG(DT_F16, DT_BF16, 4);
    else FG(DT_F16, DT_F16, 4);
  } else {
    if (a.a_dtype == DT_F32) FG(DT_BF16, DT_F32, 4);
    else FG(DT_BF16, DT_BF16, 4);
  }
#undef FG
  return hipGetLastError();
}

hipError_t launch_plain_to_frag(int ty, const void* in, int G, long gsi, int N, int Kd, void* out, long gso,
                                hipStream_t st) {
  if (Kd % 64) return hipErrorInvalidValue;
  dim3 grid(2048), block(256);
  if (ty == DT_F32)
    hipLaunchKernelGGL(plain_to_frag_kernel<DT_F32>, grid, block, 0, st, static_cast<const float*>(in), G, gsi, N, Kd,
                       static_cast<float*>(out), gso);
  else
    hipLaunchKernelGGL(plain_to_frag_kernel<DT_F16>, grid, block, 0, st, static_cast<const uint16_t*>(in), G, gsi, N,
                       Kd, static_cast<uint16_t*>(out), gso);
  return hipGetLastError();
}

hipError_t launch_tgemm(int ty, const TGemmArgs& a, hipStream_t st) {
  if (a.S <= 0 || a.M <= 0) return hipSuccess;
  if (a.N < 1 || a.N > 32 || a.M % 8 || a.lda % 8 || a.a_c0 % 8) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.M + 127) / 128), (unsigned)a.S), block(256);
#define TG(TY, SA) hipLaunchKernelGGL((tgemm_kernel<TY, SA>), grid, block, 0, st, a)
  if (ty == DT_F32) {
    TG(DT_F32, DT_F32);
  } else if (ty == DT_F16) {
    if (a.a_dtype == DT_F32) TG(DT_F16, DT_F32);
    else if (a.a_dtype == DT_BF16) TG(DT_F16, DT_BF16);
    else TG(DT_F16, DT_F16);
  } else {
    if (a.a_dtype == DT_F32) TG(DT_BF16, DT_F32);
    else TG(DT_BF16, DT_BF16);
  }
#undef TG
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

hipError_t launch_tile_scan(const int* count, int S, int rows, int* tile_off, hipStream_t st) {
  if (S < 1 || S > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, st, count, S, rows, 1, tile_off);
  return hipGetLastError();
}

int fgemm_rows(int ty) { return ty == DT_F32 ? 64 : 128; }

hipError_t launch_pad_scan(const int* count, int S, int* kpad_off, hipStream_t st) {
  if (S < 1 || S > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, st, count, S, 64, 64, kpad_off);
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

hipError_t launch_gather_assign(const AssignArgs& a, hipStream_t st) {
  if (a.Na <= 0) return hipSuccess;
  if (a.k > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_assign_kernel, dim3((a.Na + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_act(int ty, const ActArgs& a, hipStream_t st) {
  if (a.Na <= 0) return hipSuccess;
  if (a.f % 64 || a.NS < 1 || a.NS > a.f / 64 || a.Pin < 1 || a.Pin > 2) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.Na + 63) / 64 + a.E), (unsigned)a.NS), block(256);
#define AK(TY)                                                                     \
  do {                                                                             \
    if (a.Pin == 2) {                                                              \
      if (a.r) hipLaunchKernelGGL((act_kernel<TY, 2, true>), grid, block, 0, st, a);  \
      else hipLaunchKernelGGL((act_kernel<TY, 2, false>), grid, block, 0, st, a);     \
    } else {                                                                       \
      if (a.r) hipLaunchKernelGGL((act_kernel<TY, 1, true>), grid, block, 0, st, a);  \
      else hipLaunchKernelGGL((act_kernel<TY, 1, false>), grid, block, 0, st, a);     \
    }                                                                              \
  } while (0)
  // 16-bit residual layers: the expansions and column sums on MFMAs (large
  // INT4 layer 839 -> 511 us); fp32 layers keep exact fp32 sums
  if (a.r && ty != DT_F32) {
    if (ty == DT_F16) {
      if (a.Pin == 2) hipLaunchKernelGGL((act_mfma_kernel<DT_F16, 2>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((act_mfma_kernel<DT_F16, 1>), grid, block, 0, st, a);
    } else {
      if (a.Pin == 2) hipLaunchKernelGGL((act_mfma_kernel<DT_BF16, 2>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((act_mfma_kernel<DT_BF16, 1>), grid, block, 0, st, a);
    }
    return hipGetLastError();
  }
  switch (ty) {
    case DT_F32: AK(DT_F32); break;
    case DT_F16: AK(DT_F16); break;
    default: AK(DT_BF16); break;
  }
#undef AK
  return hipGetLastError();
}

hipError_t launch_act_plain(int ty, const ActArgs& a, const int* arow, float* dw, hipStream_t st) {
  if (a.Na <= 0) return hipSuccess;
  if (a.f % 4 || a.r || a.Pin < 1 || a.Pin > 2) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.Na + 3) / 4)), block(256);
#define AP(TY)                                                                                  \
  do {                                                                                          \
    if (a.Pin == 2) hipLaunchKernelGGL((act_plain_kernel<TY, 2>), grid, block, 0, st, a, arow, dw); \
    else hipLaunchKernelGGL((act_plain_kernel<TY, 1>), grid, block, 0, st, a, arow, dw);          \
  } while (0)
  switch (ty) {
    case DT_F32: AP(DT_F32); break;
    case DT_F16: AP(DT_F16); break;
    default: AP(DT_BF16); break;
  }
#undef AP
  return hipGetLastError();
}

hipError_t launch_act_finish(const float* part, int NS, int Na, int Pin, int r, const float* pw, const float* ea,
                             const int* arow, float* q, float* wu2, float* dw, hipStream_t st) {
  if (Na <= 0) return hipSuccess;
  hipLaunchKernelGGL(act_finish_kernel, dim3((Na + 3) / 4), dim3(256), 0, st, part, NS, Na, Pin, r, pw, ea, arow, q,
                     wu2, dw);
  return hipGetLastError();
}

hipError_t launch_row_sums(int ty, const void* dz, const void* wh, const int* garow, const int* apos, int R, int kg,
                           int ke, int k, int f, int Pin, void* dZbar, void* hbar, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  if (ke > MAX_SLOTS || f % 4) return hipErrorInvalidValue;
  dim3 grid(R), block(256);
  if (ty == DT_F32)
    hipLaunchKernelGGL(row_sums_kernel<DT_F32>, grid, block, 0, st, static_cast<const float*>(dz),
                       static_cast<const float*>(wh), garow, apos, kg, ke, k, f, Pin, static_cast<float*>(dZbar),
                       static_cast<float*>(hbar));
  else if (ty == DT_F16)
    hipLaunchKernelGGL(row_sums_kernel<DT_F16>, grid, block, 0, st, static_cast<const uint16_t*>(dz),
                       static_cast<const uint16_t*>(wh), garow, apos, kg, ke, k, f, Pin,
                       static_cast<uint16_t*>(dZbar), static_cast<uint16_t*>(hbar));
  else
    hipLaunchKernelGGL(row_sums_kernel<DT_BF16>, grid, block, 0, st, static_cast<const uint16_t*>(dz),
                       static_cast<const uint16_t*>(wh), garow, apos, kg, ke, k, f, Pin,
                       static_cast<uint16_t*>(dZbar), static_cast<uint16_t*>(hbar));
  return hipGetLastError();
}

hipError_t launch_tok(const TokArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (a.cols <= 0 || a.cols % 4 || a.d % 16) return hipErrorInvalidValue;
  dim3 grid(a.T, (a.d + a.cols - 1) / a.cols), block(256);
  switch (a.x_dtype) {
    case DT_F32: hipLaunchKernelGGL(tok_kernel<DT_F32>, grid, block, 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(tok_kernel<DT_F16>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(tok_kernel<DT_BF16>, grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_invert_rows(const int* garow, int R, int* grow, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(invert_rows_kernel, dim3((R + 255) / 256), dim3(256), 0, st, garow, R, grow);
  return hipGetLastError();
}

hipError_t launch_a1t(int ty, const float* Atp, int E, int Pin, int d, void* A1T, hipStream_t st) {
  dim3 grid(1024), block(256);
  if (ty == DT_F32)
    hipLaunchKernelGGL(a1t_kernel<DT_F32>, grid, block, 0, st, Atp, E, Pin, d, static_cast<float*>(A1T));
  else if (ty == DT_F16)
    hipLaunchKernelGGL(a1t_kernel<DT_F16>, grid, block, 0, st, Atp, E, Pin, d, static_cast<uint16_t*>(A1T));
  else
    hipLaunchKernelGGL(a1t_kernel<DT_BF16>, grid, block, 0, st, Atp, E, Pin, d, static_cast<uint16_t*>(A1T));
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
