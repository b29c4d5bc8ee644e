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
//         V[row, slot of j] += (w_j h_j) . A_down,j   (MFMA straight from the
//                                     registers of h, summed over the
//                                     workgroup in LDS, over column tiles by
//                                     the vreduce kernel)
//  G2 : y = [hbar | V] . [W2_base^g ; B_down stacked] -- the down projection
//       sum_j w_j h_j W~_down,j = hbar W2_base + sum_j (w_j h_j A_down,j) B_down,j^T
//       with a tail of K*16 residual k; writes Y (one group per token, one
//       k split) or fp32 partials that the combine kernel sums.
//
// Tiles: 4 wavefronts side by side along the features, 64 features (two
// 32-column blocks: for SwiGLU one gate block and its up block) each, and
// RT token blocks of 32; token rows are staged through LDS (see tile.h),
// weights read straight from their fragment-major layout.
#include <type_traits>

#include "kernels.h"
#include "tile.h"

namespace cefn {
namespace {

constexpr int CB = 2;     // feature blocks per wavefront
constexpr int BNF = 256;  // features per tile (4 wavefronts x 64)

// Tile of logical workgroup i in a 1-D grid over (group, row tile, column
// tile).  Logical order: groups in turn; inside a group, blocks of nb column
// tiles with the row tiles fastest inside a block, nb chosen so that a block
// is about one XCD's worth of workgroups (32).  Workgroups are dealt
// round-robin to the 8 XCDs (workgroup i runs on XCD i % 8), so logical
// tiles are handed to each XCD in one contiguous run: tiles that share a
// weight block or a row block run together behind the same L2.
struct TileCoord {
  int g, m0, M, nt;
};

// The group counts (G <= 256) are loaded by all lanes at once and walked
// with lane reads, so a workgroup pays one load latency here, not G.
struct GroupCounts {
  int cnt[4];
  __device__ GroupCounts(const int* gcounts, int G) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt[q] = (64 * q + lane < G) ? gcounts[64 * q + lane] : 0;
  }
  // rows of group gg (gg wave-uniform)
  __device__ int of(int gg) const {
    const int l = gg & 63;
    switch (gg >> 6) {
      case 0: return __builtin_amdgcn_readlane(cnt[0], l);
      case 1: return __builtin_amdgcn_readlane(cnt[1], l);
      case 2: return __builtin_amdgcn_readlane(cnt[2], l);
      default: return __builtin_amdgcn_readlane(cnt[3], l);
    }
  }
  __device__ int tiles(int G, int BM, int NT) const {
    int total = 0;
    for (int gg = 0; gg < G; ++gg) total += (of(gg) + BM - 1) / BM * NT;
    return total;
  }
  // logical tile L (0 <= L < tiles) -> group, first row, column tile
  __device__ bool locate(int L, int G, int BM, int NT, TileCoord& tc) const {
    for (int gg = 0; gg < G; ++gg) {
      const int Mg = of(gg);
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
};

// workgroup i of `all` -> logical tile: XCD i % 8 walks one contiguous run
__device__ __forceinline__ int xcd_order(int i, int all) {
  const int x = i & 7, j = i >> 3;
  const int q = all >> 3, rem = all & 7;
  return x * q + min(x, rem) + j;
}

// S > 1 (a k split of the down projection): the logical tiles are the S
// splits of every tile with the split outermost, so an XCD's contiguous run
// stays inside one split, where neighbouring tiles share rows or weight
// columns (the splits of one tile share nothing); *split receives it.
__device__ bool map_tile(int i, const int* gcounts, int G, int BM, int NT, TileCoord& tc, int S = 1,
                         int* split = nullptr) {
  const GroupCounts gc(gcounts, G);
  const int total = gc.tiles(G, BM, NT);
  const int all = total * S;
  if (i >= all) return false;
  int L = xcd_order(i, all);
  if (split) *split = L / total;
  return gc.locate(L % total, G, BM, NT, tc);
}

// Last-round split of the down projection.  With equal tiles, `total` tiles
// over `slots` resident workgroups leave a last round of total % slots
// tiles that keeps most compute units idle.  When at least one round is
// full and the last one is at most half full, the tiles of that last round
// (the final ones in logical order) are cut along k into S pieces each, so
// that their pieces fill the round; every piece keeps at least 4 stages and
// the pieces past the first fit in max_pieces partial tiles.
struct TailPlan {
  int F;     // tiles run whole (logical tiles 0 .. F-1)
  int tail;  // tiles F .. F+tail-1, each in S pieces
  int S;
};

__device__ __forceinline__ TailPlan tail_plan(int total, int slots, int smax, int KT, int max_pieces) {
  TailPlan p{total, 0, 1};
  if (slots <= 0 || total <= slots) return p;
  const int tail = total % slots;
  if (tail == 0 || 2 * tail > slots) return p;
  int S = min(min(smax, slots / tail), KT / 4);
  while (S > 1 && tail * (S - 1) > max_pieces) --S;
  if (S < 2) return p;
  p.F = total - tail;
  p.tail = tail;
  p.S = S;
  return p;
}

// Workgroup i under the last-round split: the first F workgroups take the
// whole tiles (XCD-aware order), the next tail * S the pieces, the pieces of
// one tile side by side.  piece: 0 .. S-1; tidx: the tile's index among the
// tail tiles (-1 for a whole tile).
__device__ bool map_tile_tail(int i, const int* gcounts, int G, int BM, int NT, int slots, int smax, int KT,
                              int max_pieces, TileCoord& tc, int& piece, int& npieces, int& tidx) {
  const GroupCounts gc(gcounts, G);
  const int total = gc.tiles(G, BM, NT);
  const TailPlan tp = tail_plan(total, slots, smax, KT, max_pieces);
  piece = 0;
  npieces = 1;
  tidx = -1;
  if (i < tp.F) return gc.locate(xcd_order(i, tp.F), G, BM, NT, tc);
  const int j = i - tp.F;
  if (j >= tp.tail * tp.S) return false;
  tidx = j / tp.S;
  piece = j - tidx * tp.S;
  npieces = tp.S;
  return gc.locate(tp.F + tidx, G, BM, NT, tc);
}

// Element v of a transposed 32x32 accumulator held by lane l: feature row
// 8 (v / 4) + 4 (l / 32) + v % 4 of the block, token column l % 32.
__device__ __forceinline__ int acc_feat(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// Store 4 consecutive features (v = 4q .. 4q+3 of one accumulator) of one
// token as one 8-byte (16-bit types) or 16-byte (fp32) write.
template <int DT>
__device__ __forceinline__ void store4(TE<DT>* p, float a, float b, float c, float d) {
  if constexpr (DT == DT_F32) {
    f4v v = {a, b, c, d};
    *reinterpret_cast<f4v*>(p) = v;
  } else {
    const uint32_t lo = static_cast<uint32_t>(from_f32<DT>(a)) | (static_cast<uint32_t>(from_f32<DT>(b)) << 16);
    const uint32_t hi = static_cast<uint32_t>(from_f32<DT>(c)) | (static_cast<uint32_t>(from_f32<DT>(d)) << 16);
    uint2 v;
    v.x = lo;
    v.y = hi;
    *reinterpret_cast<uint2*>(p) = v;
  }
}

// Main loop over the token operand TO (LDS-shared) and weight source WS
// (direct), KT >= 1 stages (d and f are multiples of 64, a k split keeps at
// least 8 stages, the residual tail is padded to 64); ends with a barrier.
// (No early exit here: one made the compiler spill the 256-token tiles.)
template <int TY, int RT, int CBT = CB, class TO, class WS>
__device__ __forceinline__ void run_tile(int KT, const TO& to, const WS& ws, int nb0, FragT<TY>* tl, int lane,
                                         f16v (&acc)[RT][CBT]) {
  // short tiles: weights two stages ahead (a stage of 32 or 64 rows has too
  // few MFMAs to cover one load's latency)
  MainloopTW<TY, RT, CBT, TO, WS, (RT <= 2 ? 2 : 1)> ml{to, ws, nb0, tl, lane};
  ml.run(KT, acc);
}

// ------------------------------------------------------------- U = X . A --
// A thin GEMM (N = K*P_in*16 columns): a workgroup takes 32 token rows x
// CB*32 columns, and its 4 wavefronts walk consecutive quarters of d for
// that same tile (rows and weights read straight into registers, two stages
// ahead), so each dependent chain is a quarter as long; the four partial
// tiles meet in LDS and wavefront c writes column block c.
template <int XT, int TY, int CB_, bool INT4, int NWU = 4>
__global__ __launch_bounds__(64 * NWU) void ugemm_kernel(GemmArgs a) {
  constexpr int BW = CB_ * 32;
  extern __shared__ __attribute__((aligned(16))) float red[];  // [NWU][CB_][16][64]
  TileCoord tc;
  if (!map_tile(blockIdx.x, a.gcounts, a.G, 32, (a.NU + BW - 1) / BW, tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wg = a.gslot ? a.gslot[g] : g;  // where the group's weights sit
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = a.goffsets[g] + m0;
  const int KT = a.d / KB;
  const int k0 = wave * KT / NWU, k1 = (wave + 1) * KT / NWU;
  TDirect<XT, TY, 1> to;
  to.init(static_cast<const TE<XT>*>(a.X) + (long)k0 * KB, a.d, lane, [&](int) -> long {
    const int m = lane & 31;
    return m0 + m < M ? (long)(a.garow[row0 + m] / a.kg) : -1L;
  });
  f16v acc[1][CB_];
  zero_acc<1, CB_>(acc);
  const int nb0 = tc.nt * CB_;
  auto run = [&](const auto& ws) {
    using WS = std::decay_t<decltype(ws)>;
    using WO = WDirect<WS, CB_>;
    WO wo;
    wo.src = ws;
    wo.nb0 = nb0;
    using TR = typename TDirect<XT, TY, 1>::Raw[1][4];
    using WR = typename WO::Raw[CB_][4];
    Mainloop<TY, 1, CB_, TDirect<XT, TY, 1>, WO, 2> ml{to, wo, lane};
    if (k1 > k0) ml.template run<TR, WR>(k1 - k0, acc);
  };
  const int KS = a.d / 16;
  if constexpr (INT4) {
    WInt4ColK<TY> ws{static_cast<const uint32_t*>(a.Bw) + wg * a.bw_gstride, a.bw_scale + wg * a.bws_gstride, KS};
    ws.ks0 = k0 * 4;
    run(ws);
  } else {
    WPlain<TY> ws{static_cast<const FragT<TY>*>(a.Bw) + wg * a.bw_gstride / 8, KS};
    ws.ks0 = k0 * 4;
    run(ws);
  }
#pragma unroll
  for (int c = 0; c < CB_; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((wave * CB_ + c) * 16 + v) * 64 + lane] = acc[0][c][v];
  __syncthreads();
  const int c = wave;
  const int m = lane & 31;
  if (c >= CB_ || m0 + m >= M || (nb0 + c) * 32 >= a.NU) return;
  TE<TY>* urow = static_cast<TE<TY>*>(a.U) + (long)(row0 + m) * a.NU + (nb0 + c) * 32 + 4 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = 4 * q + i;
      // pairwise over the wavefronts' partial tiles
      float pr[NWU];
#pragma unroll
      for (int w = 0; w < NWU; ++w) pr[w] = red[((w * CB_ + c) * 16 + v) * 64 + lane];
#pragma unroll
      for (int st = 1; st < NWU; st <<= 1)
#pragma unroll
        for (int w = 0; w + st < NWU; w += 2 * st) pr[w] += pr[w + st];
      o[i] = pr[0];
    }
    store4<TY>(urow + 8 * q, o[0], o[1], o[2], o[3]);
  }
}

// U = X . A for many rows: the tile engine (gathered rows staged through
// LDS, A straight into registers, INT4 decoded per use) on BM-row x
// CBT*128-column tiles, so a row of X is read once per 256 (CBT = 2) or 128
// (CBT = 1: twice the workgroups, for layers with under one 256-column tile
// per compute unit) columns of U rather than once per 64, and the INT4
// factors are decoded once per BM rows.
template <int XT, int TY, int RT, bool INT4, int CBT = CB>
__global__ __launch_bounds__(256, (TY != DT_F32 && RT <= 4) ? 2 : 1) void ugemm_tile_kernel(GemmArgs a) {
  constexpr int BMT = 32 * RT;
  constexpr int BNT = 4 * 32 * CBT;  // columns per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  TileCoord tc;
  if (!map_tile(blockIdx.x, a.gcounts, a.G, BMT, (a.NU + BNT - 1) / BNT, tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wg = a.gslot ? a.gslot[g] : g;  // where the group's weights sit
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nbw = (tc.nt * BNT + wave * 32 * CBT) / 32;
  const bool active = nbw * 32 < a.NU;
  const int nb0 = active ? nbw : a.NU / 32 - CBT;
  const int row0 = a.goffsets[g] + m0;
  FragT<TY>* tl = reinterpret_cast<FragT<TY>*>(smem);
  TShared<XT, TY, RT> to;
  to.init(static_cast<const TE<XT>*>(a.X), a.d, [&](int blk, int r) -> long {
    const int m = blk * 32 + r;
    return m0 + m < M ? (long)(a.garow[row0 + m] / a.kg) : -1L;
  });
  f16v acc[RT][CBT];
  zero_acc<RT, CBT>(acc);
  const int KS = a.d / 16;
  if constexpr (INT4) {
    WInt4ColK<TY> ws{static_cast<const uint32_t*>(a.Bw) + wg * a.bw_gstride, a.bw_scale + wg * a.bws_gstride, KS};
    run_tile<TY, RT, CBT>(a.d / KB, to, ws, nb0, tl, lane, acc);
  } else {
    WPlain<TY> ws{static_cast<const FragT<TY>*>(a.Bw) + wg * a.bw_gstride / 8, KS};
    run_tile<TY, RT, CBT>(a.d / KB, to, ws, nb0, tl, lane, acc);
  }
  if (!active) return;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int m = t * 32 + (lane & 31);
    if (m0 + m >= M) continue;
    TE<TY>* urow = static_cast<TE<TY>*>(a.U) + (long)(row0 + m) * a.NU + nb0 * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int c = 0; c < CBT; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store4<TY>(urow + c * 32 + 8 * q, acc[t][c][4 * q], acc[t][c][4 * q + 1], acc[t][c][4 * q + 2],
                   acc[t][c][4 * q + 3]);
  }
}

// --------------------------------------------- G1: base GEMM + epilogue --
// Residual storage of the epilogue operands: none, plain (stored in the MFMA
// type), or INT4.
enum { ER_NONE = 0, ER_PLAIN = 1, ER_INT4 = 2 };

// Raw bits of one epilogue operand fragment: plain fragments use f; INT4
// uses the 8 codes in w and its scales in x (8 fp16, or one in x[0]).  The
// field a kernel does not use is dead and takes no registers.
template <int TY>
struct ORaw {
  FragT<TY> f;
  u4v x;
  uint32_t w;
};

// Operands of one (token block, expert) step of the epilogue, loaded one
// step ahead of their use.
template <int TY, int PIN, int NFB>
struct EOps {
  ORaw<TY> b[2];      // B_j fragments of the wavefront's two feature blocks
  FragT<TY> u[PIN];   // u_j = x A_j of this lane's token, per input projection
  ORaw<TY> ad[NFB][2];  // A_down,j fragments of the wavefront's f-blocks, 2 k-steps
  float wgt;          // gate weight of expert j for this lane's token (0: not chosen)
  int slot;           // position of j in the token's chosen list (-1: not chosen)
};

// KSN = 4 or 2 (with RT = 1): for few rows per group, a workgroup owns 32
// rows x 64 * (4 / KSN) columns; its wavefronts are KSN consecutive parts
// of d times 4 / KSN column blocks of 64 (wavefront w: part w / (4 / KSN),
// block w % (4 / KSN)), rows and weights straight into registers.  The
// partial tiles of a column block meet in LDS and each of its wavefronts
// takes their sum, then the block's expert steps are dealt round-robin to
// those KSN wavefronts and their h sums meet in LDS before the store.
// KSN times the workgroups of the 256-column tiling over 4 / KSN, each
// wavefront with 1 / KSN of the dependent chain.
template <int XT, int TY, int RT, int ACT, int RES, int KSN = 0>
__global__ __launch_bounds__(256, (TY != DT_F32 && (KSN > 0 || (RT == 4 && ACT == ACT_SWIGLU))) ? 2 : 1) void gemm1_kernel(GemmArgs a) {
  constexpr bool KS = KSN > 0;
  constexpr int NCS = KS ? 4 / KSN : 1;  // column blocks of 64 per k-split tile
  static_assert(!KS || RT == 1, "the k-split tile is 32 rows");
  static_assert(KSN == 0 || KSN == 2 || KSN == 4, "d in 2 or 4 parts");
  constexpr int BMT = 32 * RT;
  constexpr int BNFT = KS ? NCS * CB * 32 : BNF;  // columns of a tile
  constexpr int PIN = (ACT == ACT_SWIGLU) ? 2 : 1;
  constexpr int NFB = (ACT == ACT_SWIGLU) ? 1 : 2;  // f-blocks per wavefront
  using F = FragT<TY>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int N = PIN * a.f;
  TileCoord tc;
  if (!map_tile(blockIdx.x, a.gcounts, a.G, BMT, (N + BNFT - 1) / BNFT, tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wg = a.gslot ? a.gslot[g] : g;  // where the group's weights sit
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ksid = wave / NCS, csid = wave % NCS;  // (KS) part of d, column block
  const int nbw = KS ? (tc.nt * NCS + csid) * CB : (tc.nt * BNF + wave * 64) / 32;
  const bool active = nbw * 32 < N;
  const int nb0 = active ? nbw : N / 32 - CB;
  // first f-block of this wavefront: SwiGLU interleaves gate and up blocks
  const int fb0 = (ACT == ACT_SWIGLU) ? nb0 / 2 : nb0;
  const int nfb = a.f / 32;
  const int row0 = a.goffsets[g] + m0;
  const int K = a.K, ke = a.ke;

  // LDS: [token stages | V sums of the current 32-token block, one slice per
  // wavefront, row stride VS = ke*16 + 1 floats (odd, so the 32 tokens of
  // one access land in different banks)] | gate weights [BMT][K] | slot of
  // expert j in the row's chosen list [BMT][K] (int8) | per token block, the
  // bit set of experts picked by any of its tokens | tile position -> row
  // of the group tile [BMT] | expert-set histogram and offsets [2][256]
  // (KS: the first region also holds the four partial tiles [4][CB][16][64]
  // floats before the V sums, and h sums [4][NFB][16][64] follow the
  // histogram)
  const int VS = ke * RPAD + 1;
  const G1Lds lay = g1_lds(KS, TY, BMT, K, ke);
  static_assert(CB == 2, "the layout counts two feature blocks per wavefront");
  float* s_v = reinterpret_cast<float*>(smem);
  float* s_w = reinterpret_cast<float*>(smem + lay.abytes);
  int8_t* s_slot = reinterpret_cast<int8_t*>(s_w + BMT * K);
  uint32_t* s_bm = reinterpret_cast<uint32_t*>(s_slot + ((BMT * K + 15) & ~15));
  int* s_perm = reinterpret_cast<int*>(s_bm + 2 * RT);
  int* s_hist = s_perm + BMT;
  float* s_h = reinterpret_cast<float*>(s_hist + 260);
  F* tl = reinterpret_cast<F*>(smem);

  for (int i = tid; i < BMT * K; i += 256) {
    s_w[i] = 0.f;
    s_slot[i] = -1;
  }
  for (int i = tid; i < 2 * RT; i += 256) s_bm[i] = 0u;
  s_hist[tid] = 0;
  __syncthreads();
  // Row order inside the tile.  With residuals, the epilogue takes one step
  // per expert picked by any token of a 32-token block, so the rows are
  // counting-sorted by the Gray-code rank of their expert set (folded to 8
  // bits; rows past the group's end last): blocks then see few distinct
  // experts.  Each token's
  // result depends only on its own column, so the order (including the
  // arbitrary order inside one key) changes no value.
  const bool mine = tid < BMT && m0 + tid < M;
  // (rows that the group sort already ordered keep their order)
  if (RES != ER_NONE && !a.rows_sorted) {
    int key = 255;
    if (mine) {
      const int t = a.garow[row0 + tid] / a.kg, ga = a.garow[row0 + tid] % a.kg;
      uint64_t set = 0;
      for (int s2 = 0; s2 < ke; ++s2) set |= 1ull << (a.idx[t * a.k + ga * ke + s2] - g * K);
      uint32_t f = static_cast<uint32_t>(set) ^ static_cast<uint32_t>(set >> 32);
      f ^= f >> 16;
      f ^= f >> 8;
      key = static_cast<int>(gray_rank8(f & 255u)) % 255;
    }
    int rk = 0;
    if (tid < BMT) rk = atomicAdd(&s_hist[key], 1);
    __syncthreads();
    // exclusive scan of the 256 bins: per wavefront, then the wave totals
    const int cnt = s_hist[tid];
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    __syncthreads();
    if (lane == 63) s_hist[256 + wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wave; ++w2) base += s_hist[256 + w2];
    s_hist[tid] = base + inc - cnt;
    __syncthreads();
    if (tid < BMT) s_perm[s_hist[key] + rk] = tid;
  } else {
    if (tid < BMT) s_perm[tid] = tid;
  }
  __syncthreads();
  for (int p = tid; p < BMT; p += 256) {
    const int i = s_perm[p];
    if (m0 + i < M) {
      const int aid = a.garow[row0 + i];
      const int t = aid / a.kg, ga = aid - t * a.kg;
      if constexpr (RES == ER_NONE) {
        // without residuals every expert of the group is the base itself:
        // sum_j w_j act(Z) = (sum_j w_j) act(Z), one step per token
        float ws = 0.f;
        for (int s = 0; s < ke; ++s) ws += a.w[t * a.k + ga * ke + s];
        s_w[p * K] = ws;
        atomicOr(&s_bm[(p >> 5) * 2], 1u);
      } else {
        for (int s = 0; s < ke; ++s) {
          const int slot = t * a.k + ga * ke + s;
          const int j = a.idx[slot] - g * K;
          s_w[p * K + j] = a.w[slot];
          s_slot[p * K + j] = static_cast<int8_t>(s);
          atomicOr(&s_bm[(p >> 5) * 2 + (j >> 5)], 1u << (j & 31));
        }
      }
    }
  }
  // (the main loop's first barrier publishes these tables)

  f16v acc[RT][CB];
  zero_acc<RT, CB>(acc);
  if constexpr (KS) {
    const int KT = a.d / KB;
    const int k0 = ksid * KT / KSN, k1 = (ksid + 1) * KT / KSN;
    using TD = TDirect<XT, TY, 1>;
    TD td;
    td.init(static_cast<const TE<XT>*>(a.X) + (long)k0 * KB, a.d, lane, [&](int) -> long {
      const int m = lane & 31;
      return m0 + m < M ? (long)(a.garow[row0 + s_perm[m]] / a.kg) : -1L;
    });
    using WO = WDirect<WPlain<TY>, CB>;
    WO wo;
    wo.src = WPlain<TY>{static_cast<const F*>(a.Bw) + wg * a.bw_gstride / 8, a.d / 16};
    wo.src.ks0 = k0 * 4;
    wo.nb0 = nb0;
    Mainloop<TY, 1, CB, TD, WO, 2> ml{td, wo, lane};
    if (k1 > k0) ml.template run<typename TD::Raw[1][4], typename WO::Raw[CB][4]>(k1 - k0, acc);
    // the partial tiles of a column block meet in LDS; each of its
    // wavefronts takes the sum
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((wave * CB + c) * 16 + v) * 64 + lane] = acc[0][c][v];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float* q = red + ((csid * CB + c) * 16 + v) * 64 + lane;
        constexpr int W = NCS * CB * 16 * 64;  // to the same block's next part
        if constexpr (KSN == 4) acc[0][c][v] = (q[0] + q[W]) + (q[2 * W] + q[3 * W]);
        else acc[0][c][v] = q[0] + q[W];
      }
    __syncthreads();
  } else {
    TShared<XT, TY, RT> to;
    to.init(static_cast<const TE<XT>*>(a.X), a.d, [&](int blk, int r) -> long {
      const int m = blk * 32 + r;
      return m0 + m < M ? (long)(a.garow[row0 + s_perm[m]] / a.kg) : -1L;
    });
    WPlain<TY> ws{static_cast<const F*>(a.Bw) + wg * a.bw_gstride / 8, a.d / 16};
    run_tile<TY, RT>(a.d / KB, to, ws, nb0, tl, lane, acc);  // ends with a barrier
  }

  // V slices, one per wavefront.  Every (token, slot) of a valid row is
  // written by exactly one expert step of each wavefront (the step of the
  // token's expert in that slot), so the steps store instead of accumulate
  // and the slices need no clearing, except an idle wavefront's (it takes
  // no steps).  With KS the steps are dealt across the wavefronts: slices
  // start at zero and accumulate (a lane owns its (token, slot, rho)
  // entries, so plain read-modify-writes need no atomics).
  // Token block t uses V set t & 1 when there are two (lay.vdb).
  if constexpr (RES != ER_NONE) {
    if constexpr (KS) {
      for (int i = tid; i < 4 * 32 * VS; i += 256) s_v[i] = 0.f;
      __syncthreads();
    } else if (!active) {
      for (int i = lane; i < 32 * VS; i += 64) {
        s_v[wave * 32 * VS + i] = 0.f;
        if (lay.vdb) s_v[(4 + wave) * 32 * VS + i] = 0.f;
      }
    }
  }
  auto vset = [&](int t) { return s_v + (lay.vdb ? (t & 1) * 4 * 32 * VS : 0); };
  const TE<TY>* Ub = static_cast<const TE<TY>*>(a.U);
  TE<TY>* H = static_cast<TE<TY>*>(a.H);
  const int h = lane >> 5;

  // expert bit sets of the token blocks (wave-uniform; idle wavefronts none)
  uint32_t mlo[RT], mhi[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    mlo[t] = active ? __builtin_amdgcn_readfirstlane(s_bm[2 * t]) : 0u;
    mhi[t] = active ? __builtin_amdgcn_readfirstlane(s_bm[2 * t + 1]) : 0u;
  }
  auto first_j = [](uint32_t lo, uint32_t hi) { return lo ? __builtin_ctz(lo) : 32 + __builtin_ctz(hi); };
  if constexpr (KS) {
    // expert steps of the block dealt round-robin over the wavefronts of a
    // column block: the r-th set bit to the one of part r % KSN
    uint32_t lo = mlo[0], hi = mhi[0], flo = 0u, fhi = 0u;
    for (int r = 0; lo | hi; ++r) {
      const int j = first_j(lo, hi);
      if (lo) lo &= lo - 1; else hi &= hi - 1;
      if ((r % KSN) == ksid) {
        if (j < 32) flo |= 1u << j; else fhi |= 1u << (j - 32);
      }
    }
    mlo[0] = flo;
    mhi[0] = fhi;
  }

  // issue the loads of step (t, j)
  auto load_ops = [&](int t, int j, EOps<TY, PIN, NFB>& o) __attribute__((always_inline)) {
    const int m = t * 32 + (lane & 31);
    const int ex = wg * K + j;
    o.wgt = s_w[m * K + j];
    o.slot = s_slot[m * K + j];
    if constexpr (RES != ER_NONE) {
      const long urow = row0 + (m0 + m < M ? s_perm[m] : 0);
#pragma unroll
      for (int p = 0; p < PIN; ++p) o.u[p] = *reinterpret_cast<const F*>(Ub + urow * a.NU + (j * PIN + p) * RPAD + 8 * h);
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int pj = (ACT == ACT_SWIGLU) ? c : 0;
        const int fb = (ACT == ACT_SWIGLU) ? fb0 : fb0 + c;
        const long fr = (long)(ex * PIN + pj) * nfb + fb;
        if constexpr (RES == ER_INT4) {
          o.b[c].w = static_cast<const uint32_t*>(a.B1)[fr * 64 + lane];
          o.b[c].x = *reinterpret_cast<const u4v*>(a.b1_scale + fr * RPAD + 8 * h);
        } else {
          o.b[c].f = static_cast<const F*>(a.B1)[fr * 64 + lane];
        }
      }
#pragma unroll
      for (int c = 0; c < NFB; ++c)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const long fr = ((long)ex * nfb + fb0 + c) * 2 + st;
          if constexpr (RES == ER_INT4) {
            const int rho = lane & 31;
            o.ad[c][st].w = static_cast<const uint32_t*>(a.Ad)[fr * 64 + lane];
            o.ad[c][st].x[0] = a.ad_scale[(fr >> 1) * RPAD + (rho < RPAD ? rho : RPAD - 1)];
          } else {
            o.ad[c][st].f = static_cast<const F*>(a.Ad)[fr * 64 + lane];
          }
        }
    }
  };

  // One expert step of token block t: takes the next expert from (lo, hi),
  // prefetches the step after it into nxt (the next expert of this block,
  // else the first of the next block, else this one again, harmlessly) and
  // computes with cur.  With INT4 operands the caller alternates the two
  // operand sets, so no operand registers are copied between steps.
  auto step = [&](auto tc_, uint32_t& lo, uint32_t& hi, const EOps<TY, PIN, NFB>& cur,
                  EOps<TY, PIN, NFB>& nxt, float (&hbar)[NFB][16], bool& have) __attribute__((always_inline)) {
    constexpr int t = decltype(tc_)::value;
    const int j = first_j(lo, hi);
    if (lo) lo &= lo - 1; else hi &= hi - 1;
    {
      int tn = t, jn = j;
      if (lo | hi) {
        jn = first_j(lo, hi);
      } else if (t + 1 < RT) {
        const int t1 = (t + 1 < RT) ? t + 1 : t;
        if (mlo[t1] | mhi[t1]) {
          tn = t1;
          jn = first_j(mlo[t1], mhi[t1]);
          have = true;
        }
      }
      load_ops(tn, jn, nxt);
    }
    f16v z[CB];
    if constexpr (RES != ER_NONE) {
      // z_j = Z + u_j B_j^T: one 16-deep MFMA step per feature block
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        F bfr;
        if constexpr (RES == ER_INT4) bfr = int4_frag_8scale<TY>(cur.b[c].w, cur.b[c].x);
        else bfr = cur.b[c].f;
        z[c] = mfma32<TY>(bfr, cur.u[(ACT == ACT_SWIGLU) ? c : 0], acc[t][c]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CB; ++c) z[c] = acc[t][c];
    }
    const float wgt = cur.wgt;
    float hw[NFB][16];
    if constexpr (ACT == ACT_SWIGLU) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        hw[0][v] = wgt * (silu_f(z[0][v]) * z[1][v]);
        hbar[0][v] += hw[0][v];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          hw[c][v] = wgt * gelu_tanh_f(z[c][v]);
          hbar[c][v] += hw[c][v];
        }
    }
    if constexpr (RES != ER_NONE) {
      // V^T[rho, token] = sum over this wavefront's features of
      // A_down[f, rho] (w h)[token, f]: the accumulator rows a lane holds
      // are the k of the MFMA, in the order the A_down operand was packed
      f16v vacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) vacc[v] = 0.f;
#pragma unroll
      for (int c = 0; c < NFB; ++c)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          F afr;
          if constexpr (RES == ER_INT4) {
            const uint16_t sb = static_cast<uint16_t>(cur.ad[c][st].x[0] & 0xFFFFu);
            afr = int4_frag_1scale<TY>(cur.ad[c][st].w, (lane & 31) < RPAD ? sb : uint16_t{0});
          } else {
            afr = cur.ad[c][st].f;
          }
          const F hfr = to_frag<TY>(&hw[c][8 * st]);  // hw is a plain float array
          vacc = mfma32<TY>(afr, hfr, vacc);
        }
      if (cur.slot >= 0) {
        float* dst = vset(t) + (wave * 32 + (lane & 31)) * VS + cur.slot * RPAD;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          if constexpr (KS) dst[acc_feat(v, lane)] += vacc[v];
          else dst[acc_feat(v, lane)] = vacc[v];
        }
      }
    }
  };

  EOps<TY, PIN, NFB> cur, nxt;
  bool have = false;  // cur already holds the first step of block t
  // (unrolled so the accumulators are indexed statically)
  static_for<RT>([&](auto tc_) __attribute__((always_inline)) {
    constexpr int t = decltype(tc_)::value;
    const int m = t * 32 + (lane & 31);  // this lane's token row in the tile
    float hbar[NFB][16];
#pragma unroll
    for (int c = 0; c < NFB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) hbar[c][v] = 0.f;
    uint32_t lo = mlo[t], hi = mhi[t];
    if ((lo | hi) && !have) load_ops(t, first_j(lo, hi), cur);
    have = false;
    while (lo | hi) {
      step(tc_, lo, hi, cur, nxt, hbar, have);
      if constexpr (RES != ER_INT4) {
        // (plain operands: the alternating form costs spills here)
        cur = nxt;
      } else {
        if (!(lo | hi)) {
          cur = nxt;  // once per block, when it took an odd number of steps
          break;
        }
        step(tc_, lo, hi, nxt, cur, hbar, have);
      }
    }
    if constexpr (KS) {
      // h sums of a column block's wavefronts meet in LDS
#pragma unroll
      for (int c = 0; c < NFB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s_h[((wave * NFB + c) * 16 + v) * 64 + lane] = hbar[c][v];
      __syncthreads();
      if (ksid == 0) {
#pragma unroll
        for (int c = 0; c < NFB; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float* q = s_h + ((csid * NFB + c) * 16 + v) * 64 + lane;
            constexpr int W = NCS * NFB * 16 * 64;
            if constexpr (KSN == 4) hbar[c][v] = (q[0] + q[W]) + (q[2 * W] + q[3 * W]);
            else hbar[c][v] = q[0] + q[W];
          }
      }
    }
    if (active && m0 + m < M && (!KS || ksid == 0)) {  // (idle wavefronts computed nothing above)
      TE<TY>* hrow = H + (long)(row0 + s_perm[m]) * a.f + 4 * h;
#pragma unroll
      for (int c = 0; c < NFB; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          store4<TY>(hrow + (fb0 + c) * 32 + 8 * q, hbar[c][4 * q], hbar[c][4 * q + 1], hbar[c][4 * q + 2],
                     hbar[c][4 * q + 3]);
    }
    if constexpr (RES != ER_NONE) {
      // the four slices of this token block -> one partial per (column tile,
      // row, slot), summed over column tiles by vreduce (KS: slices cleared)
      // (with two V sets no barrier follows: block t + 1 writes the other
      // set, and block t + 2, which writes this one, starts only after
      // every thread has passed block t + 1's barrier)
      __syncthreads();
      const int per_row = ke * RPAD;
      float* sv = vset(t);
      float* vp = a.Vp + ((long)tc.nt * a.vp_rows + row0) * per_row;
      // element e = tid + 256 i is (row r, column c) of the block; (r, c)
      // advance by a fixed step instead of a division per element
      const int rstep = 256 / per_row, cstep = 256 - rstep * per_row;
      int r = tid / per_row, c = tid - r * per_row;
      for (int e = tid; e < 32 * per_row; e += 256) {
        const int o = r * VS + c;
        const float v = (sv[o] + sv[32 * VS + o]) + (sv[2 * 32 * VS + o] + sv[3 * 32 * VS + o]);
        if constexpr (KS) sv[o] = sv[32 * VS + o] = sv[2 * 32 * VS + o] = sv[3 * 32 * VS + o] = 0.f;
        const int mr = t * 32 + r;
        if (m0 + mr < M) vp[(long)s_perm[mr] * per_row + c] = v;
        r += rstep;
        c += cstep;
        if (c >= per_row) {
          c -= per_row;
          ++r;
        }
      }
      if (!lay.vdb) __syncthreads();
    }
  });
}

// ---------------------------------------------- G2: down projection ------
// Grid: tiles x S k-splits (split s = logical workgroup % S takes stages
// [s KT / S, (s+1) KT / S) of the base part; split 0 also runs the residual
// tail).  One split and one group per token: Y is written directly;
// otherwise fp32 partials ypart[s][t*kg + ga][d] for the combine kernel.
template <int XT, int TY, int RT, bool INT4>
__global__ __launch_bounds__(256, (TY != DT_F32 && RT == 4) ? 2 : 1) void gemm2_kernel(GemmArgs a) {
  constexpr int BMT = 32 * RT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (blockIdx.x == 0 && a.zero_ptr) {
    for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;
  }
  const int NT = (a.d + BNF - 1) / BNF;
  int S = a.ksplit;
  int split = 0, tidx = -1;
  TileCoord tc;
  if (a.tail_slots > 0) {
    // (only with one k split)
    if (!map_tile_tail(blockIdx.x, a.gcounts, a.G, BMT, NT, a.tail_slots, a.tail_smax, a.f / KB,
                       a.tail_max_pieces, tc, split, S, tidx))
      return;
  } else if (!map_tile(blockIdx.x, a.gcounts, a.G, BMT, NT, tc, S, &split)) {
    return;
  }
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wg = a.gslot ? a.gslot[g] : g;  // where the group's weights sit
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nbw = (tc.nt * BNF + wave * 64) / 32;
  const bool active = nbw * 32 < a.d;
  const int nb0 = active ? nbw : a.d / 32 - CB;
  const int row0 = a.goffsets[g] + m0;
  FragT<TY>* tl = reinterpret_cast<FragT<TY>*>(smem);

  f16v acc[RT][CB];
  zero_acc<RT, CB>(acc);
  const int KT = a.f / KB;
  const int k0 = split * KT / S, k1 = (split + 1) * KT / S;
  auto rows = [&](int blk, int r) -> long {
    const int m = blk * 32 + r;
    return m0 + m < M ? (long)(row0 + m) : -1L;
  };
  {
    // hbar . W2_base^g over this split's stages
    TShared<TY, TY, RT> to;
    to.init(static_cast<const TE<TY>*>(a.H) + (long)k0 * KB, a.f, rows);
    WPlain<TY> ws{static_cast<const FragT<TY>*>(a.Bw) + wg * a.bw_gstride / 8 + (long)k0 * 4 * 64, a.f / 16};
    run_tile<TY, RT>(k1 - k0, to, ws, nb0, tl, lane, acc);
  }
  if (a.NV > 0 && split == 0) {
    // + V . [B_down,j^T]_j : 16 residual k per expert of the group
    TShared<TY, TY, RT> to;
    to.init(static_cast<const TE<TY>*>(a.V), a.NV, rows);
    const int KS = a.NV / 16;
    if constexpr (INT4) {
      WInt4Tail<TY> ws{static_cast<const uint32_t*>(a.Bd) + wg * a.bd_gstride,
                       a.bd_scale + (long)wg * a.K * (a.d / 32) * RPAD, KS, a.K, a.d / 32};
      run_tile<TY, RT>(a.NV / KB, to, ws, nb0, tl, lane, acc);
    } else {
      WPlain<TY> ws{static_cast<const FragT<TY>*>(a.Bd) + wg * a.bd_gstride / 8, KS};
      run_tile<TY, RT>(a.NV / KB, to, ws, nb0, tl, lane, acc);
    }
  }
  if (!active) return;
  if (tidx >= 0 && split > 0) {
    // a later piece of a last-round tile: the accumulators as they are
    // (register order), summed into the first piece's partials by
    // tailfix_kernel
    float* dst = a.tailpart + ((long)(tidx * (S - 1) + split - 1) * 4 + wave) * (RT * CB * 16 * 64) + lane;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[((t * CB + c) * 16 + v) * 64] = acc[t][c][v];
    return;
  }
  // (a last-round tile's first piece leaves fp32 partials for tailfix)
  const bool direct = a.kg == 1 && a.ksplit == 1 && tidx < 0;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int m = t * 32 + (lane & 31);
    if (m0 + m >= M) continue;
    const long aid = a.garow[row0 + m];
    const int n = nb0 * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v0 = acc[t][c][4 * q], v1 = acc[t][c][4 * q + 1];
        const float v2 = acc[t][c][4 * q + 2], v3 = acc[t][c][4 * q + 3];
        if (direct) {
          store4<XT>(static_cast<TE<XT>*>(a.Y) + aid * a.d + n + c * 32 + 8 * q, v0, v1, v2, v3);
        } else {
          store4<DT_F32>(a.ypart + ((long)split * a.rows_total + aid) * a.d + n + c * 32 + 8 * q, v0, v1, v2, v3);
        }
      }
  }
}

// Last-round split, second half: one workgroup per (tail tile, 32-row
// block) adds the later pieces, summed in piece order, to the partials the
// first piece wrote (same tile walk and lane mapping as the gemm2
// epilogue), into those partials or, with one chosen group, into Y.  A
// lane's 32 values of one piece are loaded together.
template <int XT, int RT>
__global__ __launch_bounds__(256) void tailfix_kernel(GemmArgs a) {
  constexpr int BMT = 32 * RT;
  constexpr int PER = RT * CB * 16 * 64;  // floats of one wavefront's partial tile
  const int NT = (a.d + BNF - 1) / BNF;
  const GroupCounts gc(a.gcounts, a.G);
  const TailPlan tp = tail_plan(gc.tiles(a.G, BMT, NT), a.tail_slots, a.tail_smax, a.f / KB, a.tail_max_pieces);
  const int tidx = blockIdx.x / RT, t = blockIdx.x - tidx * RT;
  if (tidx >= tp.tail) return;
  TileCoord tc;
  if (!gc.locate(tp.F + tidx, a.G, BMT, NT, tc)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nbw = (tc.nt * BNF + wave * 64) / 32;
  const int m = t * 32 + (lane & 31);
  if (nbw * 32 >= a.d || tc.m0 + m >= tc.M) return;
  const int S = tp.S;
  const float* src = a.tailpart + ((long)tidx * (S - 1) * 4 + wave) * PER + t * CB * 16 * 64 + lane;
  float sum[CB][16];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum[c][v] = 0.f;
  for (int p = 0; p < S - 1; ++p) {
    const float* e = src + (long)p * 4 * PER;
    float x[CB][16];
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[c][v] = e[(c * 16 + v) * 64];
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) sum[c][v] += x[c][v];
  }
  const long aid = a.garow[a.goffsets[tc.g] + tc.m0 + m];
  const int n = nbw * 32 + 4 * (lane >> 5);
  f4v y[CB][4];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) y[c][q] = *reinterpret_cast<const f4v*>(a.ypart + aid * a.d + n + c * 32 + 8 * q);
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f4v o = y[c][q];
      o[0] += sum[c][4 * q];
      o[1] += sum[c][4 * q + 1];
      o[2] += sum[c][4 * q + 2];
      o[3] += sum[c][4 * q + 3];
      if (a.kg == 1)
        store4<XT>(static_cast<TE<XT>*>(a.Y) + aid * a.d + n + c * 32 + 8 * q, o[0], o[1], o[2], o[3]);
      else
        *reinterpret_cast<f4v*>(a.ypart + aid * a.d + n + c * 32 + 8 * q) = o;
    }
}

// ------------------------------------ G2, k split inside the workgroup --
// For down projections with few rows per group: a workgroup owns RT*32 rows
// x CB_*32 columns and its 4 wavefronts walk consecutive quarters of f for
// that same tile (rows of hbar and weights straight into registers); the
// last wavefront also runs the residual tail.  The partial tiles are added
// in LDS and written once: Y directly with one group per token, else the
// per-(token, group) rows that the combine kernel sums.
template <int XT, int TY, int RT, int CB_, bool INT4>
__global__ __launch_bounds__(256) void gemm2k_kernel(GemmArgs a) {
  constexpr int NV_ = RT * CB_ * 16;  // accumulator values per lane
  extern __shared__ __attribute__((aligned(16))) float red[];  // [4 waves][NV_][64]
  if (blockIdx.x == 0 && a.zero_ptr) {
    for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;
  }
  TileCoord tc;
  if (!map_tile(blockIdx.x, a.gcounts, a.G, 32 * RT, (a.d + CB_ * 32 - 1) / (CB_ * 32), tc)) return;
  const int g = tc.g, m0 = tc.m0, M = tc.M;
  const int wg = a.gslot ? a.gslot[g] : g;  // where the group's weights sit
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = a.goffsets[g] + m0;
  const int nb0 = tc.nt * CB_;
  f16v acc[RT][CB_];
  zero_acc<RT, CB_>(acc);
  auto row_of = [&](int t) -> long {
    const int m = t * 32 + (lane & 31);
    return m0 + m < M ? (long)(row0 + m) : -1L;
  };
  auto run = [&](const TE<TY>* tbase, long ld, const auto& ws, int KT) {
    using WS = std::decay_t<decltype(ws)>;
    using TO = TDirect<TY, TY, RT>;
    using WO = WDirect<WS, CB_>;
    TO to;
    to.init(tbase, ld, lane, row_of);
    WO wo;
    wo.src = ws;
    wo.nb0 = nb0;
    using TR = typename TO::Raw[RT][4];
    using WR = typename WO::Raw[CB_][4];
    Mainloop<TY, RT, CB_, TO, WO, 1> ml{to, wo, lane};
    if (KT > 0) ml.template run<TR, WR>(KT, acc);
  };
  {
    const int KT = a.f / KB;
    const int k0 = wave * KT / 4, k1 = (wave + 1) * KT / 4;
    WPlain<TY> ws{static_cast<const FragT<TY>*>(a.Bw) + wg * a.bw_gstride / 8, a.f / 16};
    ws.ks0 = k0 * 4;
    run(static_cast<const TE<TY>*>(a.H) + (long)k0 * KB, a.f, ws, k1 - k0);
  }
  if (a.NV > 0 && wave == 3) {
    const int KS = a.NV / 16;
    if constexpr (INT4) {
      WInt4Tail<TY> ws{static_cast<const uint32_t*>(a.Bd) + wg * a.bd_gstride,
                       a.bd_scale + (long)wg * a.K * (a.d / 32) * RPAD, KS, a.K, a.d / 32};
      run(static_cast<const TE<TY>*>(a.V), a.NV, ws, a.NV / KB);
    } else {
      WPlain<TY> ws{static_cast<const FragT<TY>*>(a.Bd) + wg * a.bd_gstride / 8, KS};
      run(static_cast<const TE<TY>*>(a.V), a.NV, ws, a.NV / KB);
    }
  }
  // each wavefront parks its partial tile in its own LDS slice (plain
  // stores: adds from several wavefronts to one LDS word serialise)
  float* mine = red + (size_t)wave * NV_ * 64;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int c = 0; c < CB_; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) mine[((t * CB_ + c) * 16 + v) * 64 + lane] = acc[t][c][v];
  __syncthreads();
  // item (t, c, q) x lane: 4 consecutive features of one token
  for (int it = threadIdx.x; it < RT * CB_ * 4 * 64; it += 256) {
    const int l = it & 63, tcq = it >> 6;
    const int q = tcq & 3, c = (tcq >> 2) % CB_, t = (tcq >> 2) / CB_;
    const int m = t * 32 + (l & 31);
    const int n = (nb0 + c) * 32 + 8 * q + 4 * (l >> 5);
    if (m0 + m >= M || n >= a.d) continue;
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t e = ((size_t)(t * CB_ + c) * 16 + 4 * q + i) * 64 + l;
      o[i] = (red[e] + red[e + NV_ * 64]) + (red[e + 2 * NV_ * 64] + red[e + 3 * NV_ * 64]);
    }
    const long aid = a.garow[row0 + m];
    if (a.kg == 1) store4<XT>(static_cast<TE<XT>*>(a.Y) + aid * a.d + n, o[0], o[1], o[2], o[3]);
    else store4<DT_F32>(a.ypart + aid * a.d + n, o[0], o[1], o[2], o[3]);
  }
}

// ----------------------------------------------------------------- V sum --
// V[row, j*16 + rho] = sum over G1 column tiles of the partial for the slot
// of expert j in the row's chosen list; zero for experts the row did not
// pick.  V is stored in the MFMA type: the down projection's residual tail
// would round it to that type on load anyway.  One thread per element of V;
// eight partials of a thread in flight at a time (small layers: the most
// threads, the shortest chains).
template <int TY>
__global__ __launch_bounds__(256) void vreduce_kernel(VReduceArgs a) {
  TE<TY>* V = static_cast<TE<TY>*>(a.V);
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)a.rows * a.NV) return;
  const int row = (int)(e / a.NV), col = (int)(e % a.NV);
  const int j = col / RPAD, rho = col % RPAD;
  const int aid = a.garow[row];
  const int t = aid / a.kg, ga = aid - t * a.kg;
  const int ex = a.gidx[aid] * a.K + j;
  int sl = -1;
  for (int s = 0; s < a.ke; ++s)
    if (a.idx[t * a.k + ga * a.ke + s] == ex) sl = s;
  float sum = 0.f;
  if (sl >= 0) {
    const float* p = a.Vp + ((long)row * a.ke + sl) * RPAD + rho;
    const long step = a.vp_rows * a.ke * RPAD;
    // eight partials in flight per round (the loads are independent), the
    // eight running sums added pairwise at the end
    float q[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int nt = 0; nt < a.ntiles; nt += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = nt + u < a.ntiles ? p[(long)(nt + u) * step] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] += v[u];
    }
    sum = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
  }
  V[e] = from_f32<TY>(sum);
}

// The same sum for many rows: one thread per (row, 16-column block j; j < K
// an expert of the group, the others padding, written as zeros).  The
// row's lookups are done once for its 16 values, whose partials are 64
// contiguous bytes per column tile; four tiles' loads are in flight at a
// time, tile nt summed into running sum nt % 4, the four sums added
// pairwise at the end (large INT4 layer: 21 -> 13.5 us; on small layers
// the longer per-thread chain measured slower).
template <int TY>
__global__ __launch_bounds__(256) void vreduce_rows_kernel(VReduceArgs a) {
  TE<TY>* V = static_cast<TE<TY>*>(a.V);
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const int NJ = a.NV / RPAD;
  if (e >= (long)a.rows * NJ) return;
  const int row = (int)(e / NJ), j = (int)(e % NJ);
  const int aid = a.garow[row];
  const int t = aid / a.kg, ga = aid - t * a.kg;
  const int ex = a.gidx[aid] * a.K + j;
  int sl = -1;
  if (j < a.K)
    for (int s = 0; s < a.ke; ++s)
      if (a.idx[t * a.k + ga * a.ke + s] == ex) sl = s;
  float sum[RPAD];
#pragma unroll
  for (int r = 0; r < RPAD; ++r) sum[r] = 0.f;
  if (sl >= 0) {
    const f4v* p = reinterpret_cast<const f4v*>(a.Vp + ((long)row * a.ke + sl) * RPAD);
    const long step = a.vp_rows * a.ke * RPAD / 4;  // in f4v
    f4v q[4][RPAD / 4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < RPAD / 4; ++w) q[u][w] = f4v{0.f, 0.f, 0.f, 0.f};
    for (int nt = 0; nt < a.ntiles; nt += 4) {
      f4v v[4][RPAD / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < RPAD / 4; ++w)
          v[u][w] = nt + u < a.ntiles ? p[(long)(nt + u) * step + w] : f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < RPAD / 4; ++w) q[u][w] += v[u][w];
    }
#pragma unroll
    for (int w = 0; w < RPAD / 4; ++w) {
      const f4v s4 = (q[0][w] + q[1][w]) + (q[2][w] + q[3][w]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[4 * w + i] = s4[i];
    }
  }
  TE<TY>* out = V + (long)row * a.NV + j * RPAD;
#pragma unroll
  for (int q = 0; q < RPAD / 4; ++q) store4<TY>(out + 4 * q, sum[4 * q], sum[4 * q + 1], sum[4 * q + 2], sum[4 * q + 3]);
}

// ------------------------------------------------ bf16 -> fp16 activations --
// For bf16 activations with fp16 MFMAs, one pass converting X to fp16 (exact
// for the activations' range, the same conversion the tile loaders would
// otherwise do per stage on the path between the loads and the LDS
// commit), eight elements per thread.
__global__ __launch_bounds__(256) void cvt_bf16_f16_kernel(const u4v* in, u4v* out, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u4v v = in[i];
  u4v o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = bf16_bits_to_f32(static_cast<uint16_t>(v[q] & 0xFFFFu));
    const float hi = bf16_bits_to_f32(static_cast<uint16_t>(v[q] >> 16));
    const uint32_t l16 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(lo));
    const uint32_t h16 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hi));
    o[q] = l16 | (h16 << 16);
  }
  out[i] = o;
}

// ---------------------------------------------------------------- combine --
// Y[t] = sum over k splits s and chosen groups ga of ypart[s][t*kg + ga].
template <int XT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const long n4 = (long)a.T * a.d / 4;
  const long stride = (long)a.T * a.kg * a.d;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const long t = (i * 4) / a.d, c = (i * 4) % a.d;
    f4v s = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.ksplit; ++sp)
      for (int ga = 0; ga < a.kg; ++ga) {
        const f4v v = *reinterpret_cast<const f4v*>(a.ypart + sp * stride + (t * a.kg + ga) * a.d + c);
        s += v;
      }
    store4<XT>(static_cast<TE<XT>*>(a.Y) + t * a.d + c, s[0], s[1], s[2], s[3]);
  }
}

// ------------------------------------------------ debug: residual decode --
// Decodes one stored factor [n][r] back to values, reading the layouts the
// kernels use: kind 0 At (columns aux0 + rho, k = row permuted, KS = aux1),
// kind 1 B1 (column = row, k = rho, plain 16-deep step), kind 2 Ad,
// kind 3 Bd (column = row, k = aux0 * 16 + rho permuted, KS = aux1).
// INT4 entries are also decoded the way the GEMMs decode their operands
// (the whole 8-code fragment, in the MFMA type); an entry whose operand value
// is not its exact value rounded once to that type comes back as NaN.
__device__ __forceinline__ void perm_pos(int k, int& ks, int& h, int& e) {
  ks = (k >> 6) * 4 + ((k & 31) >> 3);
  h = (k & 63) >> 5;
  e = k & 7;
}

template <int TY>
__global__ void debug_decode_kernel(int resid, int kind, const void* src, const uint16_t* scales, long base,
                                    long sbase, int n, int r, int aux0, int aux1, float* out, int ldo) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // entry index i = row * r + rho
  if (i >= n * r) return;
  const int row = i / r, rho = i % r;
  const bool q4 = resid == RS_INT4;
  float val = 0.f;
  long fo = 0;  // fragment (word) index
  int e = 0;
  long si = 0;  // scale of this entry
  if (kind == 0) {
    const int ncol = aux0 + rho, k = row;
    int ks, h;
    perm_pos(k, ks, h, e);
    fo = (long)((ncol / 32) * aux1 + ks) * 64 + (ncol % 32) + 32 * h;
    si = sbase + ((long)(ncol / 32) * (aux1 / 2) + k / 32) * 32 + (ncol % 32);
  } else if (kind == 1) {
    const int ncol = row, h = rho / 8;
    e = rho % 8;
    fo = (long)(ncol / 32) * 64 + (ncol % 32) + 32 * h;
    si = sbase + (long)(ncol / 32) * RPAD + rho;
  } else if (kind == 2) {
    const int fb = row / 32, w = row % 32, st = w / 16, rem = w % 16;
    const int h = (rem >> 2) & 1;
    e = (rem & 3) + 4 * (rem >> 3);
    fo = ((long)fb * 2 + st) * 64 + rho + 32 * h;
    si = sbase + (long)fb * RPAD + rho;
  } else {
    const int ncol = row, k = aux0 * RPAD + rho;
    int ks, h;
    perm_pos(k, ks, h, e);
    fo = (long)((ncol / 32) * aux1 + ks) * 64 + (ncol % 32) + 32 * h;
    si = sbase + (long)(ncol / 32) * RPAD + rho;
  }
  if (q4) {
    const uint32_t word = static_cast<const uint32_t*>(src)[base + fo];
    val = int4_value(word, e, f16_bits_to_f32(scales[si]));
    if constexpr (TY != DT_F32) {
      // B1 and Bd fragments carry 8 scales (entries e' of the fragment at
      // scale index si - e + e'), At and Ad one
      FragT<TY> fr;
      if (kind == 1 || kind == 3) {
        u4v s8;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          s8[q] = static_cast<uint32_t>(scales[si - e + 2 * q]) | (static_cast<uint32_t>(scales[si - e + 2 * q + 1]) << 16);
        fr = int4_frag_8scale<TY>(word, s8);
      } else {
        fr = int4_frag_1scale<TY>(word, scales[si]);
      }
      const u4v fb = __builtin_bit_cast(u4v, fr);
      const uint32_t got = (fb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      if (got != from_f32<TY>(val)) val = __builtin_nanf("");
    }
  } else {
    val = load_as_f32<TY>(static_cast<const TE<TY>*>(src), (base + fo) * 8 + e);
  }
  out[(long)row * ldo + rho] = val;
}

// ---------------------------------------------------------------- launch --
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

// Residual storage kinds valid for a (activation type, MFMA type) pair:
// plain residuals are stored in the MFMA type (F32 with an F32 base, F16 with
// an F16 base), INT4 needs a 16-bit base.
template <int XT, int TY, int RT, int ACT, int KSN>
hipError_t launch_g1_act(const GemmArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (a.resid == RS_NONE) return go(gemm1_kernel<XT, TY, RT, ACT, ER_NONE, KSN>, grid, lds, a, st);
  if constexpr (TY == DT_F32) {
    if (a.resid == RS_F32) return go(gemm1_kernel<XT, TY, RT, ACT, ER_PLAIN, KSN>, grid, lds, a, st);
  } else {
    if (a.resid == RS_INT4) return go(gemm1_kernel<XT, TY, RT, ACT, ER_INT4, KSN>, grid, lds, a, st);
    if constexpr (TY == DT_F16) {
      if (a.resid == RS_F16) return go(gemm1_kernel<XT, TY, RT, ACT, ER_PLAIN, KSN>, grid, lds, a, st);
    }
  }
  return hipErrorInvalidValue;
}

template <int XT, int TY, int RT, int KSN = 0>
hipError_t launch_g1(const GemmArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (a.act == ACT_SWIGLU) return launch_g1_act<XT, TY, RT, ACT_SWIGLU, KSN>(a, grid, lds, st);
  if constexpr (RT <= 4) return launch_g1_act<XT, TY, RT, ACT_GELU, KSN>(a, grid, lds, st);
  return hipErrorInvalidValue;
}

template <int XT, int TY, int RT>
hipError_t launch_rt(int kind, const GemmArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = gemm_lds(kind, TY, RT * 32, a.K, a.ke);
  const bool int4 = a.resid == RS_INT4;
  switch (kind) {
    case GK_U:
      return hipErrorInvalidValue;  // launched by launch_ugemm
    case GK_UT:
      if constexpr (TY != DT_F32) {
        // under one 256-column tile per compute unit: 128-column tiles
        // (twice the workgroups; each row of X read twice)
        const unsigned nt2 = (unsigned)(a.NU + BNF - 1) / BNF, nt1 = (unsigned)(a.NU + 127) / 128;
        if (grid.x < 256 && nt1 > nt2) {
          const dim3 g1(grid.x / nt2 * nt1);
          if (int4) return go(ugemm_tile_kernel<XT, TY, RT, true, 1>, g1, lds, a, st);
          return go(ugemm_tile_kernel<XT, TY, RT, false, 1>, g1, lds, a, st);
        }
      }
      if (int4) return go(ugemm_tile_kernel<XT, TY, RT, true>, grid, lds, a, st);
      return go(ugemm_tile_kernel<XT, TY, RT, false>, grid, lds, a, st);
    case GK_G1:
      return launch_g1<XT, TY, RT>(a, grid, lds, st);
    case GK_G1K:
      if constexpr (RT == 1) return launch_g1<XT, TY, 1, 4>(a, grid, lds, st);
      return hipErrorInvalidValue;
    case GK_G1K2:
      if constexpr (RT == 1) return launch_g1<XT, TY, 1, 2>(a, grid, lds, st);
      return hipErrorInvalidValue;
    case GK_G2:
      if (int4) return go(gemm2_kernel<XT, TY, RT, true>, grid, lds, a, st);
      return go(gemm2_kernel<XT, TY, RT, false>, grid, lds, a, st);
  }
  return hipErrorInvalidValue;
}

template <int XT, int TY>
hipError_t launch_types(int kind, int bm, const GemmArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (TY == DT_F32) {
    // fp32 fragments are twice as large: small tiles only
    switch (bm) {
      case 32: return launch_rt<XT, TY, 1>(kind, a, grid, st);
      case 64: return launch_rt<XT, TY, 2>(kind, a, grid, st);
    }
  } else {
    switch (bm) {
      case 32: return launch_rt<XT, TY, 1>(kind, a, grid, st);
      case 64: return launch_rt<XT, TY, 2>(kind, a, grid, st);
      case 128: return launch_rt<XT, TY, 4>(kind, a, grid, st);
      case 256: return launch_rt<XT, TY, 8>(kind, a, grid, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t gemm_lds(int kind, int ty, int bm, int K, int ke) {
  const size_t fb = ty == DT_F32 ? 32 : 16;
  const size_t tbytes = 2 * (size_t)(bm / 32) * 4 * 64 * fb;
  if (kind != GK_G1 && kind != GK_G1K && kind != GK_G1K2) return tbytes;
  return g1_lds(kind != GK_G1, ty, bm, K, ke).total;
}

template <class KF>
hipError_t go_nw(KF kfn, dim3 grid, int nw, size_t lds, const GemmArgs& a, hipStream_t st) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kfn, grid, dim3(64 * nw), lds, st, a);
  return hipGetLastError();
}

template <int XT, int TY, int CB_, bool INT4>
hipError_t launch_ugemm_cb(const GemmArgs& a, dim3 grid, hipStream_t st) {
  // 8 wavefronts (a dependent chain half as long) when there are fewer
  // workgroups than two per compute unit and every wavefront keeps at least
  // 2 stages of d; 32- and 64-column 16-bit tiles only (the others would
  // spill at two wavefronts per SIMD)
  if constexpr (CB_ <= 2 && TY != DT_F32) {
    if (grid.x < 512 && a.d / KB >= 16)
      return go_nw(ugemm_kernel<XT, TY, CB_, INT4, 8>, grid, 8, (size_t)8 * CB_ * 16 * 64 * sizeof(float), a, st);
  }
  return go_nw(ugemm_kernel<XT, TY, CB_, INT4, 4>, grid, 4, (size_t)4 * CB_ * 16 * 64 * sizeof(float), a, st);
}

template <int XT, int TY>
hipError_t launch_ugemm_t(const GemmArgs& a, int max_mtiles, hipStream_t st) {
  const bool int4 = a.resid == RS_INT4;
  // INT4 factors are decoded per use: narrower tiles keep two workgroups per
  // compute unit to overlap the decode with the other's loads; narrower
  // tiles also when the wider ones would leave most compute units idle
  // few INT4 tiles (decode-shaped batches): 32-column tiles, twice the
  // workgroups streaming the factors (decode layer 20 -> 17.5 us)
  if (int4 && (long)max_mtiles * ((a.NU + 63) / 64) < 256) {
    const dim3 grid((unsigned)max_mtiles * ((a.NU + 31) / 32));
    return launch_ugemm_cb<XT, TY, 1, true>(a, grid, st);
  }
  if (a.NU <= 64 || int4 || (long)max_mtiles * ((a.NU + 63) / 64) < 256) {
    const dim3 grid((unsigned)max_mtiles * ((a.NU + 63) / 64));
    if (int4) return launch_ugemm_cb<XT, TY, 2, true>(a, grid, st);
    return launch_ugemm_cb<XT, TY, 2, false>(a, grid, st);
  }
  const dim3 grid((unsigned)max_mtiles * ((a.NU + 127) / 128));
  if (int4) return launch_ugemm_cb<XT, TY, 4, true>(a, grid, st);
  return launch_ugemm_cb<XT, TY, 4, false>(a, grid, st);
}

template <int XT, int TY>
hipError_t launch_g2k_t(const GemmArgs& a, int max_mtiles, hipStream_t st) {
  const bool int4 = a.resid == RS_INT4;
  const dim3 grid((unsigned)max_mtiles * ((a.d + 127) / 128));
  const size_t lds = (size_t)4 * 2 * 4 * 16 * 64 * sizeof(float);
  if (int4) return go(gemm2k_kernel<XT, TY, 2, 4, true>, grid, lds, a, st);
  return go(gemm2k_kernel<XT, TY, 2, 4, false>, grid, lds, a, st);
}

hipError_t launch_gemm(int kind, int x_dtype, int mma_dtype, int bm, const GemmArgs& a, int max_mtiles,
                       int ntiles, int splits, hipStream_t st) {
  if (max_mtiles <= 0 || ntiles <= 0) return hipSuccess;
  if (kind == GK_G2K) {
    // 64-row tiles x 128 columns: max_mtiles must be counted for bm = 64
    if (x_dtype == DT_F32 && mma_dtype == DT_F32) return launch_g2k_t<DT_F32, DT_F32>(a, max_mtiles, st);
    if (x_dtype == DT_F16 && mma_dtype == DT_F16) return launch_g2k_t<DT_F16, DT_F16>(a, max_mtiles, st);
    if (x_dtype == DT_BF16 && mma_dtype == DT_BF16) return launch_g2k_t<DT_BF16, DT_BF16>(a, max_mtiles, st);
    if (x_dtype == DT_BF16 && mma_dtype == DT_F16) return launch_g2k_t<DT_BF16, DT_F16>(a, max_mtiles, st);
    return hipErrorInvalidValue;
  }
  if (kind == GK_U) {
    // 32-row tiles: max_mtiles must be counted for bm = 32
    if (x_dtype == DT_F32 && mma_dtype == DT_F32) return launch_ugemm_t<DT_F32, DT_F32>(a, max_mtiles, st);
    if (x_dtype == DT_F16 && mma_dtype == DT_F16) return launch_ugemm_t<DT_F16, DT_F16>(a, max_mtiles, st);
    if (x_dtype == DT_BF16 && mma_dtype == DT_BF16) return launch_ugemm_t<DT_BF16, DT_BF16>(a, max_mtiles, st);
    if (x_dtype == DT_BF16 && mma_dtype == DT_F16) return launch_ugemm_t<DT_BF16, DT_F16>(a, max_mtiles, st);
    return hipErrorInvalidValue;
  }
  dim3 grid((unsigned)max_mtiles * (unsigned)ntiles * (unsigned)splits);
  if (x_dtype == DT_F32 && mma_dtype == DT_F32) return launch_types<DT_F32, DT_F32>(kind, bm, a, grid, st);
  if (x_dtype == DT_F16 && mma_dtype == DT_F16) return launch_types<DT_F16, DT_F16>(kind, bm, a, grid, st);
  if (x_dtype == DT_BF16 && mma_dtype == DT_BF16) return launch_types<DT_BF16, DT_BF16>(kind, bm, a, grid, st);
  if (x_dtype == DT_BF16 && mma_dtype == DT_F16) return launch_types<DT_BF16, DT_F16>(kind, bm, a, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_cvt_x(const void* X, void* X16, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long n8 = n / 8;  // n = T * d, d a multiple of 64
  hipLaunchKernelGGL(cvt_bf16_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const u4v*>(X), static_cast<u4v*>(X16), n8);
  return hipGetLastError();
}

hipError_t launch_vreduce(int mma_dtype, const VReduceArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  // many rows (the per-element form would take several rounds of the
  // chip): a thread per 16 values; otherwise a thread per value
  const long nblk = (long)a.rows * (a.NV / RPAD);
  if (nblk >= 65536) {
    const dim3 grid((unsigned)((nblk + 255) / 256));
    switch (mma_dtype) {
      case DT_F32: hipLaunchKernelGGL(vreduce_rows_kernel<DT_F32>, grid, dim3(256), 0, st, a); break;
      case DT_F16: hipLaunchKernelGGL(vreduce_rows_kernel<DT_F16>, grid, dim3(256), 0, st, a); break;
      case DT_BF16: hipLaunchKernelGGL(vreduce_rows_kernel<DT_BF16>, grid, dim3(256), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(((long)a.rows * a.NV + 255) / 256));
  switch (mma_dtype) {
    case DT_F32: hipLaunchKernelGGL(vreduce_kernel<DT_F32>, grid, dim3(256), 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(vreduce_kernel<DT_F16>, grid, dim3(256), 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL(vreduce_kernel<DT_BF16>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
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

template <int XT>
hipError_t launch_tailfix_t(int bm, const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.tail_slots / 2 * (bm / 32)));  // a tail is at most half a round
  switch (bm) {
    case 32: hipLaunchKernelGGL((tailfix_kernel<XT, 1>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((tailfix_kernel<XT, 2>), grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((tailfix_kernel<XT, 4>), grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL((tailfix_kernel<XT, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tailfix(int x_dtype, int bm, const GemmArgs& a, hipStream_t st) {
  if (a.tail_slots <= 0) return hipSuccess;
  switch (x_dtype) {
    case DT_F32: return launch_tailfix_t<DT_F32>(bm, a, st);
    case DT_F16: return launch_tailfix_t<DT_F16>(bm, a, st);
    case DT_BF16: return launch_tailfix_t<DT_BF16>(bm, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_debug_decode(int mma_dtype, int resid, int kind, const void* src, const uint16_t* scales,
                               long base, long sbase, int n, int r, int aux0, int aux1, float* out, int ldo,
                               hipStream_t st) {
  const int tot = n * r;
  dim3 grid((tot + 255) / 256), block(256);
  switch (mma_dtype) {
    case DT_F32: hipLaunchKernelGGL(debug_decode_kernel<DT_F32>, grid, block, 0, st, resid, kind, src, scales, base, sbase, n, r, aux0, aux1, out, ldo); break;
    case DT_F16: hipLaunchKernelGGL(debug_decode_kernel<DT_F16>, grid, block, 0, st, resid, kind, src, scales, base, sbase, n, r, aux0, aux1, out, ldo); break;
    case DT_BF16: hipLaunchKernelGGL(debug_decode_kernel<DT_BF16>, grid, block, 0, st, resid, kind, src, scales, base, sbase, n, r, aux0, aux1, out, ldo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cefn
