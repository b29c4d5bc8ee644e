// Grouped MFMA GEMMs of the compressed-expert layer.
//
// The factored expert ("Breaking the MoE LLM Trilemma", papernotes.org note,
// key design 2) is x W~_i = x W_base^g + (x A_i) B_i^T; the base product is
// the same for every expert of group g, so it is computed once per
// (token, chosen group) and reused (same section).  Rows of every GEMM here
// are the group lists built by the scatter kernel: row = position in the
// group-major list of (token, chosen group) pairs.
//
//  U  : U[row] = x . [A_{p,gK+j}]_{j<K, p<P_in}      (thin GEMM, N = K*P_in*16)
//  G1 : Z = x . W1_base^g on MFMA; epilogue per expert j of the group:
//         z_j = Z + u_j B_j^T          (one 16-deep MFMA step, C operand = Z)
//         h_j = SiLU(z_gate) * z_up    (or GELU_tanh(z))
//         hbar += w_j h_j              (gate weight w_j = 0 if row did not pick j)
//         V[row, j] += (w_j h_j) . A_down,j   (16x16x32 MFMA, atomics over column tiles)
//  G2 : y = [hbar | V] . [W2_base^g ; B_down stacked]  -- the down projection
//       sum_j w_j h_j W~_down,j = hbar W2_base + sum_j (w_j h_j A_down,j) B_down,j^T
//       with a K-tail of K*16 residual rows; writes Y (one group per token) or
//       a per-(token, group) partial that the combine kernel sums.
//
// Tiles are BM rows x 256 columns; the 4 wavefronts of a workgroup split the
// columns (64 each: one 32-column gate block and its up block for SwiGLU).
// A (activations) is staged through LDS (double-buffered, padded rows); B
// (weights) is stored fragment-major and read straight into registers one
// 64-deep stage ahead.
#include "common.h"
#include "kernels.h"

namespace cefn {
namespace {

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int APAD = 8;
constexpr int AST = BK + APAD;  // LDS row stride of the A tile, elements

template <int TY> struct Chunk { using T = u4v; };
template <> struct Chunk<DT_F32> { using T = f8; };

template <int TY> using TE = typename Elem<TY>::T;

__device__ bool find_tile(const int* gcounts, int G, int BM, int mt, int& g, int& m0, int& M) {
  int acc = 0;
  for (int gg = 0; gg < G; ++gg) {
    const int Mg = gcounts[gg];
    const int n = (Mg + BM - 1) / BM;
    if (mt < acc + n) {
      g = gg;
      m0 = (mt - acc) * BM;
      M = Mg;
      return true;
    }
    acc += n;
  }
  return false;
}

template <int TY>
__device__ __forceinline__ typename Chunk<TY>::T zero_chunk() {
  typename Chunk<TY>::T c;
  if constexpr (TY == DT_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = 0.f;
  } else {
    c[0] = c[1] = c[2] = c[3] = 0u;
  }
  return c;
}

template <int TY>
__device__ __forceinline__ typename Chunk<TY>::T chunk_from_f32(const float* v) {
  if constexpr (TY == DT_F32) {
    f8 c;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = v[i];
    return c;
  } else {
    return __builtin_bit_cast(u4v, to_frag<TY>(v));
  }
}

// 8 consecutive activations of type XT converted to an MFMA chunk of type TY.
template <int XT, int TY>
__device__ __forceinline__ typename Chunk<TY>::T load_x_chunk(const TE<XT>* p) {
  if constexpr (XT == TY) {
    if constexpr (TY == DT_F32) {
      const f4v* q = reinterpret_cast<const f4v*>(p);
      f4v a = q[0], b = q[1];
      f8 c;
      c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
      c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
      return c;
    } else {
      return *reinterpret_cast<const u4v*>(p);
    }
  } else {
    static_assert(XT == DT_BF16 && TY == DT_F16, "unsupported activation/MFMA type pair");
    u4v raw = *reinterpret_cast<const u4v*>(p);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t b = static_cast<uint16_t>((raw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      v[i] = bf16_bits_to_f32(b);
    }
    return chunk_from_f32<TY>(v);
  }
}

template <int TY>
__device__ __forceinline__ void store_chunk(TE<TY>* dst, const typename Chunk<TY>::T& c) {
  if constexpr (TY == DT_F32) {
    f4v a, b;
    a[0] = c[0]; a[1] = c[1]; a[2] = c[2]; a[3] = c[3];
    b[0] = c[4]; b[1] = c[5]; b[2] = c[6]; b[3] = c[7];
    reinterpret_cast<f4v*>(dst)[0] = a;
    reinterpret_cast<f4v*>(dst)[1] = b;
  } else {
    *reinterpret_cast<u4v*>(dst) = c;
  }
}

// ------------------------------------------------------ A-operand loaders --
// Gathered token rows of X (K axis = d).
template <int XT, int TY, int BM>
struct AGather {
  static constexpr int CPT = BM * BK / 8 / 256;
  const TE<XT>* rowp[CPT];
  int lofs[CPT];
  int kc[CPT];
  __device__ void init(const GemmArgs& a, int row0, int m0, int M) {
    const TE<XT>* X = static_cast<const TE<XT>*>(a.X);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int lr = c / (BK / 8);
      kc[j] = c % (BK / 8);
      lofs[j] = lr * AST + kc[j] * 8;
      if (m0 + lr < M) {
        const int t = a.garow[row0 + lr] / a.kg;
        rowp[j] = X + (long)t * a.d;
      } else {
        rowp[j] = nullptr;
      }
    }
  }
  __device__ void fetch(int kt, typename Chunk<TY>::T (&r)[CPT]) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      r[j] = rowp[j] ? load_x_chunk<XT, TY>(rowp[j] + kt * BK + kc[j] * 8) : zero_chunk<TY>();
  }
  __device__ void store(const typename Chunk<TY>::T (&r)[CPT], TE<TY>* buf) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) store_chunk<TY>(buf + lofs[j], r[j]);
  }
};

// Rows of [hbar | V] (K axis = f, then NV residual columns).
template <int TY, int BM>
struct AHV {
  static constexpr int CPT = BM * BK / 8 / 256;
  const TE<TY>* hrow[CPT];
  const float* vrow[CPT];
  int lofs[CPT];
  int kc[CPT];
  int f;
  __device__ void init(const GemmArgs& a, int row0, int m0, int M) {
    f = a.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int lr = c / (BK / 8);
      kc[j] = c % (BK / 8);
      lofs[j] = lr * AST + kc[j] * 8;
      if (m0 + lr < M) {
        const long row = row0 + lr;
        hrow[j] = static_cast<const TE<TY>*>(a.H) + row * a.f;
        vrow[j] = a.V ? a.V + row * a.NV : nullptr;
      } else {
        hrow[j] = nullptr;
        vrow[j] = nullptr;
      }
    }
  }
  __device__ void fetch(int kt, typename Chunk<TY>::T (&r)[CPT]) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int k0 = kt * BK + kc[j] * 8;
      if (!hrow[j]) {
        r[j] = zero_chunk<TY>();
      } else if (k0 < f) {
        r[j] = load_x_chunk<TY, TY>(hrow[j] + k0);
      } else {
        const f4v* q = reinterpret_cast<const f4v*>(vrow[j] + (k0 - f));
        f4v x0 = q[0], x1 = q[1];
        float v[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        r[j] = chunk_from_f32<TY>(v);
      }
    }
  }
  __device__ void store(const typename Chunk<TY>::T (&r)[CPT], TE<TY>* buf) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) store_chunk<TY>(buf + lofs[j], r[j]);
  }
};

// ------------------------------------------------------ B-operand loaders --
// Fragment-major matrix of type TY: block nb, global k-step ks.
template <int TY>
__device__ __forceinline__ typename Frag<TY>::T frag_at(const TE<TY>* base, int KS, int nb, int ks,
                                                        int lane) {
  return load_frag<TY>(base + ((long)(nb * KS + ks) * 64 + lane) * 8);
}

// ------------------------------------------------------------- mainloop --
template <int TY, int BM, class AL, class BL>
__device__ __forceinline__ void mainloop(int KT, const AL& al, const BL& bl, f16v (&acc)[BM / 32][2],
                                         TE<TY>* As, bool active, int lane) {
  constexpr int RB = BM / 32;
  constexpr int KSS = BK / 16;
  using Fr = typename Frag<TY>::T;
  typename Chunk<TY>::T regs[AL::CPT];
  Fr bcur[KSS][2], bnext[KSS][2];
  al.fetch(0, regs);
  al.store(regs, As);
  if (active) {
#pragma unroll
    for (int ks = 0; ks < KSS; ++ks)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) bcur[ks][cb] = bl(ks, cb);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      al.fetch(kt + 1, regs);
      if (active) {
#pragma unroll
        for (int ks = 0; ks < KSS; ++ks)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) bnext[ks][cb] = bl((kt + 1) * KSS + ks, cb);
      }
    }
    const TE<TY>* buf = As + (kt & 1) * BM * AST;
    if (active) {
#pragma unroll
      for (int ks = 0; ks < KSS; ++ks) {
        Fr af[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          af[rb] = load_frag<TY>(buf + (rb * 32 + (lane & 31)) * AST + ks * 16 + 8 * (lane >> 5));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma32<TY>(af[rb], bcur[ks][cb], acc[rb][cb]);
      }
    }
    if (more) {
      al.store(regs, As + ((kt + 1) & 1) * BM * AST);
      if (active) {
#pragma unroll
        for (int ks = 0; ks < KSS; ++ks)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) bcur[ks][cb] = bnext[ks][cb];
      }
    }
    __syncthreads();
  }
}

template <int BM>
__device__ __forceinline__ void zero_acc(f16v (&acc)[BM / 32][2]) {
#pragma unroll
  for (int rb = 0; rb < BM / 32; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.f;
}

// ------------------------------------------------------------- U = X . A --
template <int XT, int TY, int BM>
__global__ __launch_bounds__(256) void ugemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int g, m0, M;
  if (!find_tile(a.gcounts, a.G, BM, blockIdx.y, g, m0, M)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * BN + wave * 64;
  const bool active = n0 < a.NU;
  const int row0 = a.goffsets[g] + m0;
  TE<TY>* As = reinterpret_cast<TE<TY>*>(smem);

  // V rows of this tile start at zero (G1 accumulates into them)
  if (blockIdx.x == 0 && a.V) {
    const int rows = min(BM, M - m0);
    for (int i = threadIdx.x; i < rows * a.NV; i += 256) a.V[(long)(row0 + i / a.NV) * a.NV + i % a.NV] = 0.f;
  }

  AGather<XT, TY, BM> al;
  al.init(a, row0, m0, M);
  const int KS = a.d / 16;
  const int nb0 = n0 / 32;
  f16v acc[BM / 32][2];
  zero_acc<BM>(acc);
  if (a.resid == RS_INT4) {
    const uint32_t* W = static_cast<const uint32_t*>(a.Bw) + g * a.bw_gstride;
    const uint16_t* S = a.bw_scale + g * a.bws_gstride;
    const int KB = a.d / 32;
    auto bl = [&](int ks, int cb) {
      const int nb = nb0 + cb;
      const uint32_t word = W[(long)(nb * KS + ks) * 64 + lane];
      const float sc = f16_bits_to_f32(S[((long)nb * KB + (ks >> 1)) * 32 + (lane & 31)]);
      return int4_frag_1scale<TY>(word, sc);
    };
    mainloop<TY, BM>(a.d / BK, al, bl, acc, As, active, lane);
  } else {
    const TE<TY>* W = static_cast<const TE<TY>*>(a.Bw) + g * a.bw_gstride;
    auto bl = [&](int ks, int cb) { return frag_at<TY>(W, KS, nb0 + cb, ks, lane); };
    mainloop<TY, BM>(a.d / BK, al, bl, acc, As, active, lane);
  }
  if (!active) return;
  TE<TY>* U = static_cast<TE<TY>*>(a.U);
#pragma unroll
  for (int rb = 0; rb < BM / 32; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rb * 32 + acc32_row(v, lane);
        if (m0 + r < M) U[(long)(row0 + r) * a.NU + n0 + cb * 32 + (lane & 31)] = from_f32<TY>(acc[rb][cb][v]);
      }
}

// --------------------------------------------- G1: base GEMM + epilogue --
template <int XT, int TY, int BM, int ACT>
__global__ __launch_bounds__(256) void gemm1_kernel(GemmArgs a) {
  constexpr int RB = BM / 32;
  constexpr int NF = (ACT == ACT_SWIGLU) ? 1 : 2;  // 32-column f-blocks per wavefront
  constexpr int HST = NF * 32 + 8;                  // LDS row stride of the h tile
  using Fr = typename Frag<TY>::T;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int g, m0, M;
  if (!find_tile(a.gcounts, a.G, BM, blockIdx.y, g, m0, M)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int N = (ACT == ACT_SWIGLU) ? 2 * a.f : a.f;
  const int n0 = blockIdx.x * BN + wave * 64;
  const bool active = n0 < N;
  const int row0 = a.goffsets[g] + m0;
  const int K = a.K;

  // LDS: [A tiles | h tiles] (aliased) | per-row gate weights | used flags
  const size_t abytes = sizeof(TE<TY>) * 2 * BM * AST;
  const size_t hbytes = sizeof(TE<TY>) * 4 * BM * HST;
  char* p = smem + (abytes > hbytes ? abytes : hbytes);
  float* s_w = reinterpret_cast<float*>(p);
  int* s_used = reinterpret_cast<int*>(s_w + BM * K);
  TE<TY>* As = reinterpret_cast<TE<TY>*>(smem);
  TE<TY>* Hs = reinterpret_cast<TE<TY>*>(smem) + wave * BM * HST;

  for (int i = tid; i < BM * K; i += 256) s_w[i] = 0.f;
  for (int j = tid; j < K; j += 256) s_used[j] = 0;
  __syncthreads();
  for (int i = tid; i < BM; i += 256) {
    if (m0 + i < M) {
      const int aid = a.garow[row0 + i];
      const int t = aid / a.kg, ga = aid - t * a.kg;
      for (int s = 0; s < a.ke; ++s) {
        const int slot = t * a.k + ga * a.ke + s;
        const int j = a.idx[slot] - g * K;
        s_w[i * K + j] = a.w[slot];
        s_used[j] = 1;
      }
    }
  }

  AGather<XT, TY, BM> al;
  al.init(a, row0, m0, M);
  const int KS = a.d / 16;
  const int nb0 = n0 / 32;
  const TE<TY>* W = static_cast<const TE<TY>*>(a.Bw) + g * a.bw_gstride;
  auto bl = [&](int ks, int cb) { return frag_at<TY>(W, KS, nb0 + cb, ks, lane); };
  f16v acc[RB][2];
  zero_acc<BM>(acc);
  mainloop<TY, BM>(a.d / BK, al, bl, acc, As, active, lane);  // ends with a barrier

  // first 32-column f-block of this wavefront
  const int fb0 = (ACT == ACT_SWIGLU) ? n0 / 64 : n0 / 32;
  const int nfb = a.f / 32;
  f16v hbar[RB][NF];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NF; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) hbar[rb][c][v] = 0.f;

  const bool has_resid = a.resid != RS_NONE;
  const bool int4 = a.resid == RS_INT4;
  const TE<TY>* Ub = static_cast<const TE<TY>*>(a.U);
  for (int j = 0; j < K; ++j) {
    if (!s_used[j]) continue;
    const int ex = g * K + j;
    if (active) {
      // B_j fragments for this wavefront's columns (one 16-deep step)
      Fr bres[2];
      if (has_resid) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          // SwiGLU: c = projection (gate, up) of f-block fb0; GELU: f-block fb0 + c
          const int pj = (ACT == ACT_SWIGLU) ? c : 0;
          const int fb = (ACT == ACT_SWIGLU) ? fb0 : fb0 + c;
          const long fr = ((long)(ex * (NF == 1 ? 2 : 1) + pj) * nfb + fb);
          if (int4) {
            const uint32_t word = static_cast<const uint32_t*>(a.B1)[fr * 64 + lane];
            bres[c] = int4_frag_8scale<TY>(word, a.b1_scale + fr * RPAD + 8 * (lane >> 5));
          } else {
            bres[c] = load_frag<TY>(static_cast<const TE<TY>*>(a.B1) + (fr * 64 + lane) * 8);
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f16v z[2];
        const int r_lane = rb * 32 + (lane & 31);
        if (has_resid) {
          const bool rv = m0 + r_lane < M;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int pj = (ACT == ACT_SWIGLU) ? c : 0;
            Fr u = rv ? load_frag<TY>(Ub + (long)(row0 + r_lane) * a.NU + (j * (NF == 1 ? 2 : 1) + pj) * RPAD + 8 * (lane >> 5))
                      : zero_frag<TY>();
            z[c] = mfma32<TY>(u, bres[c], acc[rb][c]);
          }
        } else {
          z[0] = acc[rb][0];
          z[1] = acc[rb][1];
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = rb * 32 + acc32_row(v, lane);
          const float wgt = s_w[r * K + j];
          if constexpr (ACT == ACT_SWIGLU) {
            float hw = 0.f;
            if (wgt != 0.f) hw = wgt * (silu_f(z[0][v]) * z[1][v]);
            hbar[rb][0][v] += hw;
            if (has_resid) Hs[r * HST + (lane & 31)] = from_f32<TY>(hw);
          } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              float hw = 0.f;
              if (wgt != 0.f) hw = wgt * gelu_tanh_f(z[c][v]);
              hbar[rb][c][v] += hw;
              if (has_resid) Hs[r * HST + c * 32 + (lane & 31)] = from_f32<TY>(hw);
            }
          }
        }
      }
    }
    if (has_resid) {
      __syncthreads();
      if (active) {
        // V[row, j] += (w_j h_j)[row, this wavefront's f] . A_down,j[f, :]
#pragma unroll
        for (int mb = 0; mb < BM / 16; ++mb) {
          f4v vacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NF; ++c) {
            const Fr hf = load_frag<TY>(Hs + (mb * 16 + (lane & 15)) * HST + c * 32 + 8 * (lane >> 4));
            const long fr = (long)ex * nfb + fb0 + c;
            Fr adf;
            if (int4) {
              const uint32_t word = static_cast<const uint32_t*>(a.Ad)[fr * 64 + lane];
              adf = int4_frag_1scale<TY>(word, f16_bits_to_f32(a.ad_scale[fr * RPAD + (lane & 15)]));
            } else {
              adf = load_frag<TY>(static_cast<const TE<TY>*>(a.Ad) + (fr * 64 + lane) * 8);
            }
            vacc = mfma16<TY>(hf, adf, vacc);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = mb * 16 + acc16_row(v, lane);
            if (s_w[r * K + j] != 0.f)
              atomicAdd(a.V + (long)(row0 + r) * a.NV + j * RPAD + (lane & 15), vacc[v]);
          }
        }
      }
      __syncthreads();
    }
  }
  if (!active) return;
  TE<TY>* H = static_cast<TE<TY>*>(a.H);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NF; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rb * 32 + acc32_row(v, lane);
        if (m0 + r < M) H[(long)(row0 + r) * a.f + (fb0 + c) * 32 + (lane & 31)] = from_f32<TY>(hbar[rb][c][v]);
      }
}

// ---------------------------------------------- G2: down projection ------
template <int XT, int TY, int BM>
__global__ __launch_bounds__(256) void gemm2_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (blockIdx.x == 0 && blockIdx.y == 0 && a.zero_ptr) {
    for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;
  }
  int g, m0, M;
  if (!find_tile(a.gcounts, a.G, BM, blockIdx.y, g, m0, M)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * BN + wave * 64;
  const bool active = n0 < a.d;
  const int row0 = a.goffsets[g] + m0;
  TE<TY>* As = reinterpret_cast<TE<TY>*>(smem);

  AHV<TY, BM> al;
  al.init(a, row0, m0, M);
  const int KSm = a.f / 16;       // k-steps of the base part
  const int KSt = a.NV / 16;      // k-steps of the residual tail
  const int nb0 = n0 / 32;
  const int nd32 = a.d / 32;
  const TE<TY>* W = static_cast<const TE<TY>*>(a.Bw) + g * a.bw_gstride;
  const bool int4 = a.resid == RS_INT4;
  auto bl = [&](int ks, int cb) -> typename Frag<TY>::T {
    const int nb = nb0 + cb;
    if (ks < KSm) return frag_at<TY>(W, KSm, nb, ks, lane);
    const int kt = ks - KSm;  // residual expert j = kt (16 = one padded rank)
    if (kt >= a.K) return zero_frag<TY>();
    if (int4) {
      const uint32_t word = static_cast<const uint32_t*>(a.Bd)[g * a.bd_gstride + (long)(nb * KSt + kt) * 64 + lane];
      return int4_frag_8scale<TY>(word, a.bd_scale + ((long)(g * a.K + kt) * nd32 + nb) * RPAD + 8 * (lane >> 5));
    }
    return frag_at<TY>(static_cast<const TE<TY>*>(a.Bd) + g * a.bd_gstride, KSt, nb, kt, lane);
  };
  f16v acc[BM / 32][2];
  zero_acc<BM>(acc);
  mainloop<TY, BM>((a.f + a.NV) / BK, al, bl, acc, As, active, lane);
  if (!active) return;
#pragma unroll
  for (int rb = 0; rb < BM / 32; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = rb * 32 + acc32_row(v, lane);
      if (m0 + r >= M) continue;
      const int aid = a.garow[row0 + r];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int n = n0 + cb * 32 + (lane & 31);
        if (a.kg == 1) {
          static_cast<TE<XT>*>(a.Y)[(long)aid * a.d + n] = from_f32<XT>(acc[rb][cb][v]);
        } else {
          a.ypart[(long)aid * a.d + n] = acc[rb][cb][v];
        }
      }
    }
}

// ---------------------------------------------------------------- combine --
template <int XT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const long n4 = (long)a.T * a.d / 4;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const long t = (i * 4) / a.d, c = (i * 4) % a.d;
    f4v s = *reinterpret_cast<const f4v*>(a.ypart + (t * a.kg) * a.d + c);
    for (int ga = 1; ga < a.kg; ++ga) {
      f4v v = *reinterpret_cast<const f4v*>(a.ypart + (t * a.kg + ga) * a.d + c);
      s += v;
    }
    TE<XT>* Y = static_cast<TE<XT>*>(a.Y) + t * a.d + c;
#pragma unroll
    for (int q = 0; q < 4; ++q) Y[q] = from_f32<XT>(s[q]);
  }
}

// ------------------------------------------------ debug: residual decode --
// kind 0: fragment-major 32x16 blocks (N = n rows of the factor's column
// space); kind 1: B1 / Bd layouts (8 scales per lane); kind 2: Ad layout.
// Writes values [n][r] of one factor.
template <int TY>
__global__ void debug_decode_kernel(int resid, int kind, const void* src, const uint16_t* scales,
                                    long base, long sbase, int n, int r, int aux0, int aux1,
                                    float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // entry index i = row * r + rho
  if (i >= n * r) return;
  const int row = i / r, rho = i % r;
  float val = 0.f;
  if (kind == 0) {
    // At: column n_col = aux0 + rho, k = row; KS = aux1 (= d/16)
    const int ncol = aux0 + rho, k = row;
    const int nb = ncol / 32, ks = k / 16, ln = (ncol % 32) + 32 * ((k % 16) / 8), e = k % 8;
    const long fo = (long)(nb * aux1 + ks) * 64 + ln;
    if (resid == RS_INT4) {
      const uint32_t word = static_cast<const uint32_t*>(src)[base + fo];
      const float sc = f16_bits_to_f32(scales[sbase + ((long)nb * (aux1 / 2) + ks / 2) * 32 + (ncol % 32)]);
      val = int4_value(word, e, sc);
    } else {
      val = load_as_f32<TY>(static_cast<const TE<TY>*>(src), (base + fo) * 8 + e);
    }
  } else if (kind == 1) {
    // B1/Bd: column = row (output index), k = aux0 * RPAD + rho; KS = aux1
    const int ncol = row, k = aux0 * RPAD + rho;
    const int nb = ncol / 32, ks = k / 16, ln = (ncol % 32) + 32 * ((k % 16) / 8), e = k % 8;
    const long fo = (long)(nb * aux1 + ks) * 64 + ln;
    if (resid == RS_INT4) {
      const uint32_t word = static_cast<const uint32_t*>(src)[base + fo];
      const float sc = f16_bits_to_f32(scales[sbase + (long)nb * RPAD + rho]);
      val = int4_value(word, e, sc);
    } else {
      val = load_as_f32<TY>(static_cast<const TE<TY>*>(src), (base + fo) * 8 + e);
    }
  } else {
    // Ad: k = row (f index), column rho
    const int fb = row / 32, ln = rho + 16 * ((row % 32) / 8), e = row % 8;
    const long fo = (long)fb * 64 + ln;
    if (resid == RS_INT4) {
      const uint32_t word = static_cast<const uint32_t*>(src)[base + fo];
      const float sc = f16_bits_to_f32(scales[sbase + (long)fb * RPAD + rho]);
      val = int4_value(word, e, sc);
    } else {
      val = load_as_f32<TY>(static_cast<const TE<TY>*>(src), (base + fo) * 8 + e);
    }
  }
  out[i] = val;
}

// ---------------------------------------------------------------- launch --
size_t gemm_lds(int kind, int ty, int bm, int K) {
  const size_t es = ty == DT_F32 ? 4 : 2;
  const size_t abytes = es * 2 * bm * AST;
  if (kind != GK_G1) return abytes;
  const size_t hbytes = es * 4 * bm * (2 * 32 + 8);
  return (abytes > hbytes ? abytes : hbytes) + sizeof(float) * bm * K + sizeof(int) * K + 64;
}

template <class KF>
hipError_t go(KF kfn, dim3 grid, size_t lds, const GemmArgs& a, hipStream_t st) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kfn, grid, dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int XT, int TY, int BM>
hipError_t launch_t(int kind, const GemmArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = gemm_lds(kind, TY, BM, a.K);
  switch (kind) {
    case GK_U: return go(ugemm_kernel<XT, TY, BM>, grid, lds, a, st);
    case GK_G1:
      if (a.act == ACT_SWIGLU) return go(gemm1_kernel<XT, TY, BM, ACT_SWIGLU>, grid, lds, a, st);
      return go(gemm1_kernel<XT, TY, BM, ACT_GELU>, grid, lds, a, st);
    case GK_G2: return go(gemm2_kernel<XT, TY, BM>, grid, lds, a, st);
  }
  return hipErrorInvalidValue;
}

template <int XT, int TY>
hipError_t launch_bm(int kind, int bm, const GemmArgs& a, dim3 grid, hipStream_t st) {
  switch (bm) {
    case 32: return launch_t<XT, TY, 32>(kind, a, grid, st);
    case 64: return launch_t<XT, TY, 64>(kind, a, grid, st);
    case 128: return launch_t<XT, TY, 128>(kind, a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int kind, int x_dtype, int mma_dtype, int bm, const GemmArgs& a,
                       int max_mtiles, int ntiles, hipStream_t st) {
  if (max_mtiles <= 0 || ntiles <= 0) return hipSuccess;
  dim3 grid(ntiles, max_mtiles);
  if (x_dtype == DT_F32 && mma_dtype == DT_F32) return launch_bm<DT_F32, DT_F32>(kind, bm, a, grid, st);
  if (x_dtype == DT_F16 && mma_dtype == DT_F16) return launch_bm<DT_F16, DT_F16>(kind, bm, a, grid, st);
  if (x_dtype == DT_BF16 && mma_dtype == DT_BF16) return launch_bm<DT_BF16, DT_BF16>(kind, bm, a, grid, st);
  if (x_dtype == DT_BF16 && mma_dtype == DT_F16) return launch_bm<DT_BF16, DT_F16>(kind, bm, a, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(int x_dtype, const CombineArgs& a, hipStream_t st) {
  const long n4 = (long)a.T * a.d / 4;
  if (n4 <= 0) return hipSuccess;
  long blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  switch (x_dtype) {
    case DT_F32: hipLaunchKernelGGL(combine_kernel<DT_F32>, dim3(blocks), dim3(256), 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(combine_kernel<DT_F16>, dim3(blocks), dim3(256), 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL(combine_kernel<DT_BF16>, dim3(blocks), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_debug_decode(int mma_dtype, int resid, int kind, const void* src,
                               const uint16_t* scales, long base, long sbase, int n, int r,
                               int aux0, int aux1, float* out, hipStream_t st) {
  const int tot = n * r;
  dim3 grid((tot + 255) / 256), block(256);
  switch (mma_dtype) {
    case DT_F32: hipLaunchKernelGGL(debug_decode_kernel<DT_F32>, grid, block, 0, st, resid, kind, src, scales, base, sbase, n, r, aux0, aux1, out); break;
    case DT_F16: hipLaunchKernelGGL(debug_decode_kernel<DT_F16>, grid, block, 0, st, resid, kind, src, scales, base, sbase, n, r, aux0, aux1, out); break;
    case DT_BF16: hipLaunchKernelGGL(debug_decode_kernel<DT_BF16>, grid, block, 0, st, resid, kind, src, scales, base, sbase, n, r, aux0, aux1, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cefn
