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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace cefn {
namespace {

constexpr int BN = 256;
constexpr int APAD = 8;  // LDS row padding of the A tile, elements (16 bytes)

template <int TY> struct Chunk { using T = u4v; };
template <> struct Chunk<DT_F32> { using T = f8; };

template <int TY> using TE = typename Elem<TY>::T;

// Tile of workgroup blockIdx.x in a 1-D grid over (group, row tile, column
// tile).  Logical order: groups in turn; inside a group, blocks of nb column
// tiles with the row tiles fastest inside a block, nb chosen so that a block
// is about one XCD's worth of workgroups (32).  Workgroups are dealt
// round-robin to the 8 XCDs (workgroup i runs on XCD i % 8), so logical
// tiles are handed to each XCD in one contiguous run: tiles that share a
// weight block or a row block run together behind the same L2.
struct TileCoord {
  int g, m0, M, nt;
};

__device__ bool map_tile(const int* gcounts, int G, int BM, int NT, TileCoord& tc) {
  int total = 0;
  for (int gg = 0; gg < G; ++gg) total += (gcounts[gg] + BM - 1) / BM * NT;
  const int i = blockIdx.x;
  if (i >= total) return false;
  const int x = i & 7, j = i >> 3;
  const int q = total >> 3, rem = total & 7;
  int L = x * q + min(x, rem) + j;
  for (int gg = 0; gg < G; ++gg) {
    const int Mg = gcounts[gg];
    const int mt = (Mg + BM - 1) / BM;
    if (L < mt * NT) {
      const int nb = max(1, 32 / mt);
      const int blk = L / (mt * nb);
      const int within = L - blk * mt * nb;
      tc.g = gg;
      tc.M = Mg;
      tc.m0 = (within % mt) * BM;
      tc.nt = blk * nb + within / mt;
      return true;
    }
    L -= mt * NT;
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
// Raw 8-element chunk of a source of type DT (16 bytes, or 32 for fp32).
template <int DT> struct Raw8 { using T = u4v; };
template <> struct Raw8<DT_F32> { using T = f8; };

template <int DT>
__device__ __forceinline__ typename Raw8<DT>::T load_raw8(const TE<DT>* p) {
  if constexpr (DT == DT_F32) {
    const f4v* q = reinterpret_cast<const f4v*>(p);
    f4v a = q[0], b = q[1];
    f8 c;
    c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
    return c;
  } else {
    return *reinterpret_cast<const u4v*>(p);
  }
}

// Convert a raw chunk of type SRC to an MFMA chunk of type TY.
template <int SRC, int TY>
__device__ __forceinline__ typename Chunk<TY>::T convert8(const typename Raw8<SRC>::T& r) {
  if constexpr (SRC == TY) {
    return r;
  } else if constexpr (SRC == DT_F32) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = r[i];
    return chunk_from_f32<TY>(v);
  } else {
    static_assert(SRC == DT_BF16 && TY == DT_F16, "unsupported activation/MFMA type pair");
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t b = static_cast<uint16_t>((r[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      v[i] = bf16_bits_to_f32(b);
    }
    return chunk_from_f32<TY>(v);
  }
}

// A-operand loader over rows of a [rows][ld] matrix of type SRC, staged to
// LDS as type TY.  fetch() only issues the loads; store() converts, zeroes
// rows past the tile's end and writes LDS, so no instruction waits on a
// load until the stage's MFMAs have been issued.  GATHER: row r of the tile
// is token garow[row0 + r] / kg of X (stride d); otherwise rows row0 + r of
// base (stride ld).
template <int SRC, int TY, int BM, int BK, bool GATHER>
struct ALoader {
  static constexpr int CPT = BM * BK / 8 / 256;
  static constexpr int AST = BK + APAD;
  using Raw = typename Raw8<SRC>::T;
  const TE<SRC>* rowp[CPT];
  int lofs[CPT];
  bool ok[CPT];
  __device__ void init(const TE<SRC>* base, long ld, const int* garow, int kg, int row0, int m0,
                       int M) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int lr = c / (BK / 8);
      const int kc = c % (BK / 8);
      lofs[j] = lr * AST + kc * 8;
      ok[j] = m0 + lr < M;
      const int r = row0 + (ok[j] ? lr : 0);
      const long src_row = GATHER ? (long)(garow[r] / kg) : (long)r;
      rowp[j] = base + src_row * ld + kc * 8;
    }
  }
  __device__ void fetch(int kt, Raw (&r)[CPT]) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) r[j] = load_raw8<SRC>(rowp[j] + kt * BK);
  }
  __device__ void store(const Raw (&r)[CPT], TE<TY>* buf) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const typename Chunk<TY>::T c = convert8<SRC, TY>(r[j]);
      store_chunk<TY>(buf + lofs[j], ok[j] ? c : zero_chunk<TY>());
    }
  }
};

// ------------------------------------------------------ B-operand loaders --
// Each loader has load(ks, cb) -> Raw (loads only) and decode(Raw) -> Frag.

// Fragment-major matrix of type TY: block nb0 + cb, k-step ks.
template <int TY>
struct BFrag {
  using Raw = typename Frag<TY>::T;
  const TE<TY>* base;
  int KS, nb0, lane;
  __device__ Raw load(int ks, int cb) const {
    return load_frag<TY>(base + ((long)((nb0 + cb) * KS + ks) * 64 + lane) * 8);
  }
  __device__ typename Frag<TY>::T decode(const Raw& r) const { return r; }
};

// INT4 fragment-major factor with one scale per lane (blocks along k):
// scales [N/32][Kd/32][32].
template <int TY>
struct BInt4K {
  struct Raw {
    uint32_t word;
    uint16_t sc;
  };
  const uint32_t* words;
  const uint16_t* scales;
  int KS, nb0, lane;
  __device__ Raw load(int ks, int cb) const {
    const int nb = nb0 + cb;
    Raw r;
    r.word = words[(long)(nb * KS + ks) * 64 + lane];
    r.sc = scales[((long)nb * (KS / 2) + (ks >> 1)) * 32 + (lane & 31)];
    return r;
  }
  __device__ typename Frag<TY>::T decode(const Raw& r) const {
    return int4_frag_1scale<TY>(r.word, f16_bits_to_f32(r.sc));
  }
};

// INT4 residual tail of the down projection (k-step kt = expert kt of the
// group, blocks along n): 8 scales per lane, scales [E][d/32][16].
template <int TY>
struct BInt4Tail {
  struct Raw {
    uint32_t word;
    u4v sc;
  };
  const uint32_t* words;
  const uint16_t* scales;  // of expert g*K
  int KS, nb0, lane, K, nd32;
  __device__ Raw load(int kt, int cb) const {
    const int nb = nb0 + cb;
    const int je = kt < K ? kt : K - 1;  // padding steps hold zero codes
    Raw r;
    r.word = words[(long)(nb * KS + kt) * 64 + lane];
    r.sc = *reinterpret_cast<const u4v*>(scales + ((long)je * nd32 + nb) * RPAD + 8 * (lane >> 5));
    return r;
  }
  __device__ typename Frag<TY>::T decode(const Raw& r) const {
    return int4_frag_8scale<TY>(r.word, r.sc);
  }
};

// ------------------------------------------------------------- mainloop --
// KS_total 16-deep k-steps (a multiple of BK / 16) in stages of BK.  Two
// register sets for B and two LDS buffers for A alternate (the loop body is
// unrolled by two so no set is copied): the loads of stage kt+1 are issued
// before stage kt's MFMAs, and their conversion, decoding and LDS stores
// come after, so the load latency overlaps the stage's MFMAs.
template <int TY, int BM, int BK, class AL, class BL>
__device__ __forceinline__ void mainloop_stage(int kt, int KT, const AL& al, const BL& bl,
                                               f16v (&acc)[BM / 32][2], TE<TY>* As, int lane,
                                               typename AL::Raw (&regs)[AL::CPT],
                                               const typename BL::Raw (&bcur)[BK / 16][2],
                                               typename BL::Raw (&bnext)[BK / 16][2]) {
  constexpr int RB = BM / 32;
  constexpr int KSS = BK / 16;
  constexpr int AST = BK + APAD;
  using Fr = typename Frag<TY>::T;
  const int kn = (kt + 1 < KT) ? kt + 1 : kt;  // the last stage re-reads itself
  al.fetch(kn, regs);
#pragma unroll
  for (int ks = 0; ks < KSS; ++ks)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) bnext[ks][cb] = bl.load(kn * KSS + ks, cb);
  // keep the next stage's loads ahead of this stage's MFMAs (left alone,
  // the scheduler sinks them next to their uses and the latency shows)
  __builtin_amdgcn_sched_barrier(0);
  const TE<TY>* buf = As + (kt & 1) * BM * AST;
#pragma unroll
  for (int ks = 0; ks < KSS; ++ks) {
    Fr af[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      af[rb] = load_frag<TY>(buf + (rb * 32 + (lane & 31)) * AST + ks * 16 + 8 * (lane >> 5));
    Fr bf[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) bf[cb] = bl.decode(bcur[ks][cb]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma32<TY>(af[rb], bf[cb], acc[rb][cb]);
  }
  __builtin_amdgcn_sched_barrier(0);
  al.store(regs, As + ((kt + 1) & 1) * BM * AST);
  __syncthreads();
}

template <int TY, int BM, int BK, class AL, class BL>
__device__ __forceinline__ void mainloop(int KS_total, const AL& al, const BL& bl,
                                         f16v (&acc)[BM / 32][2], TE<TY>* As, int lane) {
  constexpr int KSS = BK / 16;
  const int KT = KS_total / KSS;
  typename AL::Raw regs[AL::CPT];
  typename BL::Raw b0[KSS][2], b1[KSS][2];
  al.fetch(0, regs);
#pragma unroll
  for (int ks = 0; ks < KSS; ++ks)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) b0[ks][cb] = bl.load(ks, cb);
  al.store(regs, As);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    mainloop_stage<TY, BM, BK>(kt, KT, al, bl, acc, As, lane, regs, b0, b1);
    mainloop_stage<TY, BM, BK>(kt + 1, KT, al, bl, acc, As, lane, regs, b1, b0);
  }
  if (kt < KT) mainloop_stage<TY, BM, BK>(kt, KT, al, bl, acc, As, lane, regs, b0, b1);
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
template <int XT, int TY, int BM, int BK>
__global__ __launch_bounds__(256) void ugemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  TileCoord tc;
  if (!map_tile(a.gcounts, a.G, BM, (a.NU + BN - 1) / BN, tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = tc.nt * BN + wave * 64;
  const bool active = n0 < a.NU;
  const int row0 = a.goffsets[g] + m0;
  TE<TY>* As = reinterpret_cast<TE<TY>*>(smem);

  ALoader<XT, TY, BM, BK, true> al;
  al.init(static_cast<const TE<XT>*>(a.X), a.d, a.garow, a.kg, row0, m0, M);
  const int KS = a.d / 16;
  const int nb0 = (active ? n0 : a.NU - 64) / 32;  // idle wavefronts read a valid block
  f16v acc[BM / 32][2];
  zero_acc<BM>(acc);
  if (a.resid == RS_INT4) {
    BInt4K<TY> bl{static_cast<const uint32_t*>(a.Bw) + g * a.bw_gstride, a.bw_scale + g * a.bws_gstride,
                  KS, nb0, lane};
    mainloop<TY, BM, BK>(KS, al, bl, acc, As, lane);
  } else {
    BFrag<TY> bl{static_cast<const TE<TY>*>(a.Bw) + g * a.bw_gstride, KS, nb0, lane};
    mainloop<TY, BM, BK>(KS, al, bl, acc, As, lane);
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
// Per-expert operands of the G1 epilogue for one wavefront.
template <int TY, int RB, int NF>
struct ExpertOps {
  typename Frag<TY>::T b[2];       // B_j fragments (gate, up) or (f-block 0, 1)
  typename Frag<TY>::T u[RB][2];   // u_j = x A_j rows of this tile (gate, up)
  typename Frag<TY>::T ad[NF];     // A_down,j fragments of this wavefront's f-blocks
};

template <int XT, int TY, int BM, int BK, int ACT>
__global__ __launch_bounds__(256) void gemm1_kernel(GemmArgs a) {
  constexpr int RB = BM / 32;
  constexpr int NF = (ACT == ACT_SWIGLU) ? 1 : 2;  // 32-column f-blocks per wavefront
  constexpr int PIN = (ACT == ACT_SWIGLU) ? 2 : 1;
  constexpr int HST = NF * 32 + 8;                  // LDS row stride of the h tile
  constexpr int AST = BK + APAD;
  using Fr = typename Frag<TY>::T;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int N = PIN * a.f;
  TileCoord tc;
  if (!map_tile(a.gcounts, a.G, BM, (N + BN - 1) / BN, tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = tc.nt * BN + wave * 64;
  const bool active = n0 < N;
  const int row0 = a.goffsets[g] + m0;
  const int K = a.K;

  // LDS: [A tiles | h tiles] (aliased) | gate weights [BM][K] | slot of
  // expert j in the row's chosen list [BM][K] | used flags [K] | partial
  // V of the 4 wavefronts [4][BM][16]
  const size_t abytes = sizeof(TE<TY>) * 2 * BM * AST;
  const size_t hbytes = sizeof(TE<TY>) * 4 * BM * HST;
  char* p = smem + (abytes > hbytes ? abytes : hbytes);
  float* s_w = reinterpret_cast<float*>(p);
  int* s_slot = reinterpret_cast<int*>(s_w + BM * K);
  int* s_used = s_slot + BM * K;
  float* s_red = reinterpret_cast<float*>(s_used + ((K + 3) & ~3));
  TE<TY>* As = reinterpret_cast<TE<TY>*>(smem);
  TE<TY>* Hs = reinterpret_cast<TE<TY>*>(smem) + wave * BM * HST;

  for (int i = tid; i < BM * K; i += 256) {
    s_w[i] = 0.f;
    s_slot[i] = -1;
  }
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
        s_slot[i * K + j] = s;
        s_used[j] = 1;
      }
    }
  }

  ALoader<XT, TY, BM, BK, true> al;
  al.init(static_cast<const TE<XT>*>(a.X), a.d, a.garow, a.kg, row0, m0, M);
  const int KS = a.d / 16;
  const int nb0 = (active ? n0 : N - 64) / 32;  // idle wavefronts read a valid block
  BFrag<TY> bl{static_cast<const TE<TY>*>(a.Bw) + g * a.bw_gstride, KS, nb0, lane};
  f16v acc[RB][2];
  zero_acc<BM>(acc);
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

  // loads of expert j's epilogue operands (issued one expert ahead)
  auto load_ops = [&](int j, ExpertOps<TY, RB, NF>& o) {
    const int ex = g * K + j;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // SwiGLU: c = projection (gate, up) of f-block fb0; GELU: f-block fb0 + c
      const int pj = (ACT == ACT_SWIGLU) ? c : 0;
      const int fb = (ACT == ACT_SWIGLU) ? fb0 : fb0 + c;
      const long fr = (long)(ex * PIN + pj) * nfb + fb;
      if (int4) {
        const uint32_t word = static_cast<const uint32_t*>(a.B1)[fr * 64 + lane];
        o.b[c] = int4_frag_8scale<TY>(word, *reinterpret_cast<const u4v*>(a.b1_scale + fr * RPAD + 8 * (lane >> 5)));
      } else {
        o.b[c] = load_frag<TY>(static_cast<const TE<TY>*>(a.B1) + (fr * 64 + lane) * 8);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r_lane = rb * 32 + (lane & 31);
      const bool rv = m0 + r_lane < M;
      const long urow = row0 + (rv ? r_lane : 0);
#pragma unroll
      for (int c = 0; c < PIN; ++c) {
        const Fr u = load_frag<TY>(Ub + urow * a.NU + (j * PIN + c) * RPAD + 8 * (lane >> 5));
        o.u[rb][c] = rv ? u : zero_frag<TY>();
      }
    }
#pragma unroll
    for (int c = 0; c < NF; ++c) {
      const long fr = (long)ex * nfb + fb0 + c;
      if (int4) {
        const uint32_t word = static_cast<const uint32_t*>(a.Ad)[fr * 64 + lane];
        o.ad[c] = int4_frag_1scale<TY>(word, f16_bits_to_f32(a.ad_scale[fr * RPAD + (lane & 15)]));
      } else {
        o.ad[c] = load_frag<TY>(static_cast<const TE<TY>*>(a.Ad) + (fr * 64 + lane) * 8);
      }
    }
  };
  auto next_used = [&](int j) {
    while (j < K && !s_used[j]) ++j;
    return j;
  };

  // the first expert's operands do not depend on the main loop: their
  // loads are in flight during it
  ExpertOps<TY, RB, NF> cur, nxt;
  __syncthreads();  // s_used is complete
  int j = next_used(0);
  if (has_resid && active && j < K) load_ops(j, cur);
  mainloop<TY, BM, BK>(KS, al, bl, acc, As, lane);  // ends with a barrier

  while (j < K) {
    const int jn = next_used(j + 1);
    if (has_resid && active && jn < K) load_ops(jn, nxt);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this expert's work
    if (active) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f16v z[2];
        if (has_resid) {
#pragma unroll
          for (int c = 0; c < 2; ++c) z[c] = mfma32<TY>(cur.u[rb][(ACT == ACT_SWIGLU) ? c : 0], cur.b[c], acc[rb][c]);
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
            // the two rows this register holds: skip when neither picked j
            if (__any(wgt != 0.f)) {
              const float h = silu_f(z[0][v]) * z[1][v];
              hw = (wgt != 0.f) ? wgt * h : 0.f;
            }
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
      // (w_j h_j)[row, this wavefront's f] . A_down,j[f, :], summed over the
      // 4 wavefronts in LDS: one partial per (column tile, row, slot)
#pragma unroll
      for (int mb = 0; mb < BM / 16; ++mb) {
        f4v vacc = {0.f, 0.f, 0.f, 0.f};
        if (active) {
#pragma unroll
          for (int c = 0; c < NF; ++c) {
            const Fr hf = load_frag<TY>(Hs + (mb * 16 + (lane & 15)) * HST + c * 32 + 8 * (lane >> 4));
            vacc = mfma16<TY>(hf, cur.ad[c], vacc);
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s_red[(wave * BM + mb * 16 + acc16_row(v, lane)) * RPAD + (lane & 15)] = vacc[v];
      }
      __syncthreads();
      for (int e = tid; e < BM * RPAD; e += 256) {
        const int r = e / RPAD, rho = e % RPAD;
        const int sl = s_slot[r * K + j];
        if (sl >= 0) {
          const float sum = (s_red[e] + s_red[BM * RPAD + e]) +
                            (s_red[2 * BM * RPAD + e] + s_red[3 * BM * RPAD + e]);
          a.Vp[(((long)tc.nt * a.vp_rows + row0 + r) * a.ke + sl) * RPAD + rho] = sum;
        }
      }
      __syncthreads();
    }
    cur = nxt;
    j = jn;
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
template <int XT, int TY, int BM, int BK>
__global__ __launch_bounds__(256) void gemm2_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (blockIdx.x == 0 && a.zero_ptr) {
    for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;
  }
  TileCoord tc;
  if (!map_tile(a.gcounts, a.G, BM, (a.d + BN - 1) / BN, tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = tc.nt * BN + wave * 64;
  const bool active = n0 < a.d;
  const int row0 = a.goffsets[g] + m0;
  TE<TY>* As = reinterpret_cast<TE<TY>*>(smem);

  const int KSm = a.f / 16;       // k-steps of the base part
  const int KSt = a.NV / 16;      // k-steps of the residual tail
  const int nb0 = (active ? n0 : a.d - 64) / 32;  // idle wavefronts read a valid block
  const int nd32 = a.d / 32;
  f16v acc[BM / 32][2];
  zero_acc<BM>(acc);
  {
    // hbar . W2_base^g
    ALoader<TY, TY, BM, BK, false> al;
    al.init(static_cast<const TE<TY>*>(a.H), a.f, nullptr, 1, row0, m0, M);
    BFrag<TY> bl{static_cast<const TE<TY>*>(a.Bw) + g * a.bw_gstride, KSm, nb0, lane};
    mainloop<TY, BM, BK>(KSm, al, bl, acc, As, lane);
  }
  if (KSt > 0) {
    // + V . [B_down,j^T]_j : one 16-deep k-step per expert of the group
    ALoader<DT_F32, TY, BM, 64, false> al;
    al.init(a.V, a.NV, nullptr, 1, row0, m0, M);
    if (a.resid == RS_INT4) {
      BInt4Tail<TY> bl{static_cast<const uint32_t*>(a.Bd) + g * a.bd_gstride,
                       a.bd_scale + (long)g * a.K * nd32 * RPAD, KSt, nb0, lane, a.K, nd32};
      mainloop<TY, BM, 64>(KSt, al, bl, acc, As, lane);
    } else {
      BFrag<TY> bl{static_cast<const TE<TY>*>(a.Bd) + g * a.bd_gstride, KSt, nb0, lane};
      mainloop<TY, BM, 64>(KSt, al, bl, acc, As, lane);
    }
  }
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

// ----------------------------------------------------------------- V sum --
// V[row, j*16 + rho] = sum over G1 column tiles of the partial for the slot
// of expert j in the row's chosen list; zero for experts the row did not
// pick.  One block of 256 threads per 16 rows.
__global__ __launch_bounds__(256) void vreduce_kernel(VReduceArgs a) {
  const int row_base = blockIdx.x * 16;
  const int nrow = min(16, a.rows - row_base);
  if (nrow <= 0) return;
  for (int e = threadIdx.x; e < nrow * a.NV; e += 256) a.V[(long)row_base * a.NV + e] = 0.f;
  __syncthreads();
  const int per_row = a.ke * RPAD;
  for (int e = threadIdx.x; e < nrow * per_row; e += 256) {
    const int r = e / per_row, rem = e % per_row, sl = rem / RPAD, rho = rem % RPAD;
    const int row = row_base + r;
    const int aid = a.garow[row];
    const int t = aid / a.kg, ga = aid - t * a.kg;
    const int g = a.gidx[aid];
    const int j = a.idx[t * a.k + ga * a.ke + sl] - g * a.K;
    float sum = 0.f;
    for (int nt = 0; nt < a.ntiles; ++nt)
      sum += a.Vp[(((long)nt * a.vp_rows + row) * a.ke + sl) * RPAD + rho];
    a.V[(long)row * a.NV + j * RPAD + rho] = sum;
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
size_t gemm_lds(int kind, int ty, int bm, int bk, int K) {
  const size_t es = ty == DT_F32 ? 4 : 2;
  const size_t abytes = es * 2 * bm * (bk + APAD);
  if (kind != GK_G1) return abytes;
  const size_t hbytes = es * 4 * bm * (2 * 32 + 8);
  return (abytes > hbytes ? abytes : hbytes) + (sizeof(float) + sizeof(int)) * bm * K +
         sizeof(int) * ((K + 3) & ~3) + sizeof(float) * 4 * bm * RPAD + 64;
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

template <int XT, int TY, int BM, int BK>
hipError_t launch_t(int kind, const GemmArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = gemm_lds(kind, TY, BM, BK, a.K);
  switch (kind) {
    case GK_U: return go(ugemm_kernel<XT, TY, BM, BK>, grid, lds, a, st);
    case GK_G1:
      if (a.act == ACT_SWIGLU) return go(gemm1_kernel<XT, TY, BM, BK, ACT_SWIGLU>, grid, lds, a, st);
      return go(gemm1_kernel<XT, TY, BM, BK, ACT_GELU>, grid, lds, a, st);
    case GK_G2: return go(gemm2_kernel<XT, TY, BM, BK>, grid, lds, a, st);
  }
  return hipErrorInvalidValue;
}

template <int XT, int TY>
hipError_t launch_bm(int kind, int bm, int bk, const GemmArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (TY == DT_F32) {
    // fp32 fragments are twice as large: small tiles only
    if (bk != 64) return hipErrorInvalidValue;
    switch (bm) {
      case 32: return launch_t<XT, TY, 32, 64>(kind, a, grid, st);
      case 64: return launch_t<XT, TY, 64, 64>(kind, a, grid, st);
    }
    return hipErrorInvalidValue;
  } else {
    if (bk == 64) {
      switch (bm) {
        case 32: return launch_t<XT, TY, 32, 64>(kind, a, grid, st);
        case 64: return launch_t<XT, TY, 64, 64>(kind, a, grid, st);
        case 128: return launch_t<XT, TY, 128, 64>(kind, a, grid, st);
      }
    } else if (bk == 128) {
      switch (bm) {
        case 32: return launch_t<XT, TY, 32, 128>(kind, a, grid, st);
        case 64: return launch_t<XT, TY, 64, 128>(kind, a, grid, st);
        case 128: return launch_t<XT, TY, 128, 128>(kind, a, grid, st);
      }
    }
    return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm(int kind, int x_dtype, int mma_dtype, int bm, int bk, const GemmArgs& a,
                       int max_mtiles, int ntiles, hipStream_t st) {
  if (max_mtiles <= 0 || ntiles <= 0) return hipSuccess;
  dim3 grid((unsigned)max_mtiles * (unsigned)ntiles);
  if (x_dtype == DT_F32 && mma_dtype == DT_F32) return launch_bm<DT_F32, DT_F32>(kind, bm, bk, a, grid, st);
  if (x_dtype == DT_F16 && mma_dtype == DT_F16) return launch_bm<DT_F16, DT_F16>(kind, bm, bk, a, grid, st);
  if (x_dtype == DT_BF16 && mma_dtype == DT_BF16) return launch_bm<DT_BF16, DT_BF16>(kind, bm, bk, a, grid, st);
  if (x_dtype == DT_BF16 && mma_dtype == DT_F16) return launch_bm<DT_BF16, DT_F16>(kind, bm, bk, a, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_vreduce(const VReduceArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(vreduce_kernel, dim3((a.rows + 15) / 16), dim3(256), 0, st, a);
  return hipGetLastError();
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
