// MFMA tile engine shared by the grouped GEMMs.
//
// Orientation.  Every GEMM here multiplies token rows (activations, the "T"
// side) by weight columns (the "W" side) over a depth k.  The accumulators
// are held transposed: acc[t][c] is the 32x32 block of feature block c
// (rows) by token block t (columns), produced by
//   acc[t][c] = mfma(W fragment of block c, T fragment of block t, acc[t][c]).
// In that layout lane l owns one token (l % 32) of the block and 16 of its
// features, which is what the epilogues want: per-token gate weights are one
// value per lane, and h can feed the next MFMA straight from registers.
//
// k order.  Inside every 64-deep k block, k-step s (0..3) of an MFMA
// fragment gives lane half h (= lane / 32) element i the depth
//   k = 64 * kb + 32 * h + 8 * s + i,
// so over one 64-deep stage a lane reads 32 consecutive k of its row: 64
// contiguous bytes of a 16-bit token row, one full 128-byte line per row
// for the two lane halves.  Weights are packed with the same order (the
// contraction does not care how k is enumerated as long as both sides agree).
//
// Workgroup = 4 wavefronts arranged WM (token direction) x WN (feature
// direction); each wavefront computes RT token blocks x CB feature blocks.
// An operand shared by several wavefronts (T when WN > 1, W when WM > 1) is
// staged through LDS, double-buffered, one barrier per 64-deep stage; an
// operand private to a wavefront is loaded straight into registers one stage
// ahead.
#pragma once
#include "common.h"

namespace cefn {

constexpr int KB = 64;  // depth of one stage / one permuted k block

template <int TY> using TE = typename Elem<TY>::T;
template <int TY> using FragT = typename Frag<TY>::T;

// ------------------------------------------------------------ raw chunks --
// Raw16<SRC>: the 8 source elements of one fragment as loaded (16 bytes for
// 16-bit types, 32 for fp32).
template <int SRC> struct Raw16 { using T = u4v; };
template <> struct Raw16<DT_F32> { using T = f8; };
template <int SRC> using RawT = typename Raw16<SRC>::T;

template <int SRC>
__device__ __forceinline__ RawT<SRC> ld_raw(const TE<SRC>* p) {
  if constexpr (SRC == DT_F32) {
    const f4v* q = reinterpret_cast<const f4v*>(p);
    const f4v a = q[0], b = q[1];
    f8 c;
    c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
    return c;
  } else {
    return *reinterpret_cast<const u4v*>(p);
  }
}

template <int SRC>
__device__ __forceinline__ RawT<SRC> zero_raw() {
  RawT<SRC> c;
  if constexpr (SRC == DT_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = 0.f;
  } else {
    c[0] = c[1] = c[2] = c[3] = 0u;
  }
  return c;
}

// Raw chunk of type SRC -> MFMA fragment of type TY.
template <int SRC, int TY>
__device__ __forceinline__ FragT<TY> cvt_frag(const RawT<SRC>& r) {
  if constexpr (SRC == TY) {
    if constexpr (TY == DT_F32) return r;
    else return __builtin_bit_cast(FragT<TY>, r);
  } else if constexpr (SRC == DT_F32) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = r[i];
    return to_frag<TY>(v);
  } else {
    static_assert(SRC == DT_BF16 && TY == DT_F16, "unsupported activation / MFMA type pair");
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t b = static_cast<uint16_t>((r[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      v[i] = bf16_bits_to_f32(b);
    }
    return to_frag<TY>(v);
  }
}

template <int TY>
__device__ __forceinline__ void st_frag(FragT<TY>* p, const FragT<TY>& f) { *p = f; }

// ------------------------------------------------------ token operand (T) --
// Rows of a row-major [rows][ld] matrix of type SRC, optionally gathered
// (row r of the tile is source row map(r)).
//
// TDirect: a wavefront loads its own RT blocks into registers; lane l owns
// one 64-byte (128-byte for fp32) segment per stage: token row l % 32 of a
// block, k half l / 32.
// TShared: the workgroup copies all NB token blocks of a stage into LDS.
// Four consecutive lanes read the four 16-byte pieces of one 64-byte half
// row, so a load instruction covers 8 whole 128-byte lines (one cache tag
// per 64 bytes; the fragment-order mapping touched 64 tags per
// instruction, and the vector L1 tag rate then bounded the main loop).
// The LDS image is fragment-major with a swizzle: fragment (block, k-step s)
// holds logical lane L (token row r = L % 32, k half h = L / 32) in slot
// L ^ (s + 4h + 8 (r & 1)).  A store instruction's 16 lanes cover two rows
// x both k halves x the four k-steps: the s term spreads a lane quad's
// four pieces, the h term the other half of the row (32 slots on, the same
// banks without it), the r term the next row, so the 16 pieces land in 16
// different groups of 4 banks; each 16 lanes of a read take 16 consecutive
// slots, permuted.  A reader of k-step s takes slot lane ^ (s + 4h + 8 (r & 1)).
template <int SRC, int TY, int RT>
struct TDirect {
  using Raw = RawT<SRC>;
  const TE<SRC>* rowp[RT];
  bool ok[RT];
  // row_of(t): source row of token (block t, row lane % 32), or -1
  template <class RowOf>
  __device__ void init(const TE<SRC>* base, long ld, int lane, RowOf row_of) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const long r = row_of(t);
      ok[t] = r >= 0;
      rowp[t] = base + (ok[t] ? r : 0) * ld + 32 * (lane >> 5);
    }
  }
  __device__ void fetch(int kt, Raw (&r)[RT][4]) const {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) r[t][s] = ld_raw<SRC>(rowp[t] + kt * KB + 8 * s);
  }
  __device__ FragT<TY> frag(const Raw (&r)[RT][4], int t, int s) const {
    return ok[t] ? cvt_frag<SRC, TY>(r[t][s]) : zero_frag<TY>();
  }
};

template <int SRC, int TY, int NB>
struct TShared {
  // load instructions per thread and stage (64 half rows each)
  static constexpr int SEG = NB;
  using Raw = RawT<SRC>;
  const TE<SRC>* rowp[SEG];
  bool ok[SEG];
  int lofs[SEG];  // LDS fragment slot of the thread's piece
  // row_of(blk, r): source row of token r of block blk, or -1 (zeros)
  template <class RowOf>
  __device__ void init(const TE<SRC>* base, long ld, RowOf row_of) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, sq = lane & 3;
#pragma unroll
    for (int q = 0; q < SEG; ++q) {
      const int hr = (q * 4 + wave) * 16 + (lane >> 2);  // half row: 2 row + k half
      const int row = hr >> 1, hh = hr & 1, blk = row >> 5, r = row & 31;
      const long src = row_of(blk, r);
      ok[q] = src >= 0;
      rowp[q] = base + (ok[q] ? src : 0) * ld + 32 * hh + 8 * sq;
      lofs[q] = (blk * 4 + sq) * 64 + ((32 * hh + r) ^ (sq + 4 * hh + 8 * (r & 1)));
    }
  }
  __device__ void fetch(int kt, Raw (&r)[SEG]) const {
#pragma unroll
    for (int q = 0; q < SEG; ++q) r[q] = ld_raw<SRC>(rowp[q] + kt * KB);
  }
  // the first (h = 0) or second half of the instructions (the interleaved
  // main loop spreads a stage's loads over two k-steps)
  __device__ void fetch_half(int kt, int h, Raw (&r)[SEG]) const {
    constexpr int H0 = (SEG + 1) / 2;
#pragma unroll
    for (int q = 0; q < SEG; ++q)
      if ((q < H0) == (h == 0)) r[q] = ld_raw<SRC>(rowp[q] + kt * KB);
  }
  __device__ void commit(const Raw (&r)[SEG], FragT<TY>* buf) const {
#pragma unroll
    for (int q = 0; q < SEG; ++q) st_frag<TY>(buf + lofs[q], ok[q] ? cvt_frag<SRC, TY>(r[q]) : zero_frag<TY>());
  }
  // slot of logical lane `lane` in fragment (block, k-step s)
  __device__ static int slot(int lane, int s) { return lane ^ (s + 4 * (lane >> 5) + 8 * (lane & 1)); }
  static constexpr int frags_per_stage = NB * 4 * 64;
};

// ----------------------------------------------------- weight operand (W) --
// Fragment-major weights: [N/32][Kd/16][64 lanes] fragments (k permuted as
// above), so 32 columns x one 64-deep stage is 4 consecutive fragments.
// WFrag: plain TY fragments.  WInt4: 8 nibbles per lane plus scales, decoded
// by a functor (scale layout differs by matrix).
// ks0: first k-step of the range a caller walks (k-split kernels).
template <int TY>
struct WPlain {
  using Raw = FragT<TY>;
  const FragT<TY>* base;  // block 0 of this matrix
  int KS;                 // k-steps (Kd / 16)
  int ks0 = 0;
  __device__ Raw load(int nb, int kstep, int lane) const {
    return base[((long)nb * KS + ks0 + kstep) * 64 + lane];
  }
  __device__ FragT<TY> decode(const Raw& r, int, int, int) const { return r; }
};

// INT4 with one scale per (column, 32 consecutive k): scales [N/32][Kd/32][32].
// Over one 64-deep stage lane half h covers k 32h..32h+31 -- one scale.
template <int TY>
struct WInt4ColK {
  struct Raw {
    uint32_t w;
    uint16_t s;
  };
  const uint32_t* words;
  const uint16_t* scales;
  int KS;
  int ks0 = 0;
  __device__ Raw load(int nb, int kstep, int lane) const {
    kstep += ks0;
    Raw r;
    r.w = words[((long)nb * KS + kstep) * 64 + lane];
    r.s = scales[((long)nb * (KS / 2) + 2 * (kstep >> 2) + (lane >> 5)) * 32 + (lane & 31)];
    return r;
  }
  __device__ FragT<TY> decode(const Raw& r, int, int, int) const {
    return int4_frag_1scale<TY>(r.w, r.s);
  }
};

// INT4 stacked residual tail of the down projection: k = j*16 + rho (j the
// expert of the group, permuted in 64-deep blocks like every k); 8 scales per
// lane, scales [E][d/32][16] of expert gK + j.
template <int TY>
struct WInt4Tail {
  struct Raw {
    uint32_t w;
    u4v s;
  };
  const uint32_t* words;
  const uint16_t* scales;  // of expert gK
  int KS, K, nd32;
  __device__ Raw load(int nb, int kstep, int lane) const {
    // k-step kstep = 4 kb + s covers, for lane half h, expert j = 4kb + 2h + s/2
    // and rho = 8 (s % 2) + i
    const int kb = kstep >> 2, s = kstep & 3;
    int j = 4 * kb + 2 * (lane >> 5) + (s >> 1);
    j = j < K ? j : K - 1;  // padding k holds zero codes
    Raw r;
    r.w = words[((long)nb * KS + kstep) * 64 + lane];
    r.s = *reinterpret_cast<const u4v*>(scales + ((long)j * nd32 + nb) * RPAD + 8 * (s & 1));
    return r;
  }
  __device__ FragT<TY> decode(const Raw& r, int, int, int) const { return int4_frag_8scale<TY>(r.w, r.s); }
};

// WDirect: a wavefront loads CB column blocks (nb0 .. nb0 + CB - 1) itself.
template <class WS, int CB>
struct WDirect {
  using Raw = typename WS::Raw;
  WS src;
  int nb0;
  __device__ void fetch(int kt, int lane, Raw (&r)[CB][4]) const {
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int s = 0; s < 4; ++s) r[c][s] = src.load(nb0 + c, kt * 4 + s, lane);
  }
};


// ---------------------------------------------------------------- mainloop --
// Both operands straight into registers (each wavefront its own token and
// weight blocks), KT stages of 64 k.  PD: how many stages ahead the global
// loads run.  Per stage: the loads of stage kt + PD are issued first (stages
// past the end re-issue the last one, harmlessly, so no load sits in a
// branch), then the 4 k-steps of MFMAs.  Register sets rotate through a ring
// of U = PD + 1 (the loop is unrolled U times so every index is static).
template <int TY, int RT, int CB, class TO, class WO, int PD = 1>
struct Mainloop {
  static constexpr int U = PD + 1;
  using F = FragT<TY>;
  const TO& to;
  const WO& wo;
  int lane;

  template <class TR, class WR>
  __device__ __forceinline__ void frags(int s, const TR& tr, const WR& wr, F (&tf)[RT], F (&wf)[CB]) const {
#pragma unroll
    for (int t = 0; t < RT; ++t) tf[t] = to.frag(tr, t, s);
#pragma unroll
    for (int c = 0; c < CB; ++c) wf[c] = wo.src.decode(wr[c][s], 0, 0, 0);
  }

  template <int u, class TR, class WR>
  __device__ __forceinline__ void stage(int kt, int KT, f16v (&acc)[RT][CB], TR (&tr)[U], WR (&wr)[U]) const {
    constexpr int fs = (u + PD) % U;  // ring slot of stage kt + PD
    const int kn = (kt + PD < KT) ? kt + PD : KT - 1;
    to.fetch(kn, tr[fs]);
    wo.fetch(kn, lane, wr[fs]);
    __builtin_amdgcn_sched_barrier(0);
    F tf[2][RT], wf[2][CB];
    frags(0, tr[u], wr[u], tf[0], wf[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) frags(s + 1, tr[u], wr[u], tf[(s + 1) & 1], wf[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[t][c] = mfma32<TY>(wf[s & 1][c], tf[s & 1][t], acc[t][c]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  template <class TR, class WR>
  __device__ void run(int KT, f16v (&acc)[RT][CB]) const {
    TR tr[U];
    WR wr[U];
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int kn = p < KT ? p : KT - 1;
      to.fetch(kn, tr[p]);
      wo.fetch(kn, lane, wr[p]);
    }
    int kt = 0;
    for (; kt + U <= KT; kt += U) {
      stage<0>(kt, KT, acc, tr, wr);
      stage<1>(kt + 1, KT, acc, tr, wr);
      if constexpr (U > 2) stage<2>(kt + 2, KT, acc, tr, wr);
      if constexpr (U > 3) stage<3>(kt + 3, KT, acc, tr, wr);
    }
    if (kt < KT) stage<0>(kt, KT, acc, tr, wr);
    if constexpr (U > 2) {
      if (kt + 1 < KT) stage<1>(kt + 1, KT, acc, tr, wr);
    }
    if constexpr (U > 3) {
      if (kt + 2 < KT) stage<2>(kt + 2, KT, acc, tr, wr);
    }
  }
};

// ------------------------------------------------- interleaved main loop --
// Token rows staged through LDS (TShared, all 4 wavefronts share them) and
// weights loaded straight into registers (each wavefront its own CB column
// blocks).  One 64-deep stage is 4 k-steps of RT x CB MFMAs; around them:
//   k-step 0: LDS reads of k-step 1, token loads of the next stage (k-steps
//             0-1), weights of the next stage (k-step 0)
//   k-step 1: LDS reads of k-step 2, token loads (k-steps 2-3), weights (1)
//   k-step 2: LDS reads of k-step 3, weights (k-steps 2-3)
//   then the token commit into the other LDS buffer and the barrier, after
//   which k-step 3's MFMAs cover the LDS reads of the next stage's k-step 0.
// Group scheduling barriers spread each k-step's loads between its MFMAs
// rather than issuing them in one burst.  The barrier orders LDS only, so
// global loads stay in flight across it.  Ends with a full barrier (callers
// reuse the LDS).  KT >= 1.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// WPD: how many stages ahead the weights are loaded (2 for short tiles, whose
// stage of MFMAs is too short to cover the memory latency).
template <int TY, int RT, int CB, class TO, class WS, int WPD = 1>
struct MainloopTW {
  using F = FragT<TY>;
  using WR = typename WS::Raw;
  static constexpr int FPS = TO::frags_per_stage;
  static constexpr int M_MFMA = 0x008, M_VMEM = 0x020, M_DSR = 0x100;
  const TO& to;
  const WS& ws;
  int nb0;
  F* tl;
  int lane;

  __device__ __forceinline__ void mfmas(const WR (&wr)[CB][4], const F (&tf)[RT], int s, f16v (&acc)[RT][CB]) const {
    F wf[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) wf[c] = ws.decode(wr[c][s], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[t][c] = mfma32<TY>(wf[c], tf[t], acc[t][c]);
  }
  __device__ __forceinline__ void dsr(int b, int s, F (&tf)[RT]) const {
#pragma unroll
    for (int t = 0; t < RT; ++t) tf[t] = tl[b * FPS + (t * 4 + s) * 64 + TO::slot(lane, s)];
  }
  __device__ __forceinline__ void wload(int kt, int s, WR (&wr)[CB][4]) const {
#pragma unroll
    for (int c = 0; c < CB; ++c) wr[c][s] = ws.load(nb0 + c, kt * 4 + s, lane);
  }
  template <int NV>
  __device__ __forceinline__ static void pattern() {
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      __builtin_amdgcn_sched_group_barrier(M_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(M_DSR, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      __builtin_amdgcn_sched_group_barrier(M_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(M_VMEM, 1, 0);
    }
  }

  // stage kt from LDS buffer kt & 1 with weights wc; loads the tokens of
  // stage kt + 1 (clamped: the last stage reloads itself into the idle
  // buffer) and the weights of stage kt + WPD (clamped) into wn
  template <class TR>
  __device__ __forceinline__ void stage(int kt, int KT, TR& tr, WR (&wc)[CB][4], WR (&wn)[CB][4], F (&tf)[2][RT],
                                        f16v (&acc)[RT][CB]) const {
    const int b = kt & 1;
    const int kn = kt + 1 < KT ? kt + 1 : KT - 1;
    const int kw = kt + WPD < KT ? kt + WPD : KT - 1;
    dsr(b, 1, tf[1]);
    to.fetch_half(kn, 0, tr);
    wload(kw, 0, wn);
    mfmas(wc, tf[0], 0, acc);
    pattern<(TO::SEG + 1) / 2 + CB>();
    __builtin_amdgcn_sched_barrier(0);
    dsr(b, 2, tf[0]);
    to.fetch_half(kn, 1, tr);
    wload(kw, 1, wn);
    mfmas(wc, tf[1], 1, acc);
    pattern<TO::SEG / 2 + CB>();
    __builtin_amdgcn_sched_barrier(0);
    dsr(b, 3, tf[1]);
    wload(kw, 2, wn);
    wload(kw, 3, wn);
    mfmas(wc, tf[0], 2, acc);
    pattern<2 * CB>();
    __builtin_amdgcn_sched_barrier(0);
    to.commit(tr, tl + (b ^ 1) * FPS);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    dsr(b ^ 1, 0, tf[0]);
    mfmas(wc, tf[1], 3, acc);
    pattern<0>();
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ void run(int KT, f16v (&acc)[RT][CB]) const {
    static_assert(WPD == 1 || WPD == 2, "weights one or two stages ahead");
    constexpr int U = WPD + 1;  // weight register sets in the ring
    typename TO::Raw tr[TO::SEG];
    WR wr[U][CB][4];
    F tf[2][RT];
    to.fetch(0, tr);
#pragma unroll
    for (int p = 0; p < WPD; ++p)
#pragma unroll
      for (int s = 0; s < 4; ++s) wload(p < KT ? p : KT - 1, s, wr[p]);
    to.commit(tr, tl);
    lds_barrier();
    dsr(0, 0, tf[0]);
    int kt = 0;
    for (; kt + U <= KT; kt += U) {
      stage(kt, KT, tr, wr[0], wr[WPD % U], tf, acc);
      stage(kt + 1, KT, tr, wr[1], wr[(1 + WPD) % U], tf, acc);
      if constexpr (U > 2) stage(kt + 2, KT, tr, wr[2 % U], wr[(2 + WPD) % U], tf, acc);
    }
    if (kt < KT) stage(kt, KT, tr, wr[0], wr[WPD % U], tf, acc);
    if constexpr (U > 2) {
      if (kt + 1 < KT) stage(kt + 1, KT, tr, wr[1], wr[(1 + WPD) % U], tf, acc);
    }
    __syncthreads();
  }
};

template <int RT, int CB>
__device__ __forceinline__ void zero_acc(f16v (&acc)[RT][CB]) {
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][c][v] = 0.f;
}

}  // namespace cefn
