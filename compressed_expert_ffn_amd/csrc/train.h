// Internal interface of the backward-pass kernels (train.hip) used by
// backward.hip.  All matrices the backward GEMMs read are row-major with the
// contraction index k contiguous ("k-major"), in the MFMA type TY unless
// noted; k ranges are padded to multiples of 64 with zeros.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cefn {

// C[m][n] = sum_k A(m, k) B(n, k) over segments of rows (mode R) or of k
// (mode K); fp32 C.
//  mode R: segment s owns rows [seg_start[s], seg_start[s] + seg_count[s])
//          of C (row-major, ldc); A row m of the segment is a_map ? source
//          row a_map[seg_start[s] + m] / a_div : seg_start[s] + m of A
//          (lda, type a_dtype, converted to TY on load); B = b + s * b_sstride
//          ([N][K], ldb = K); K fixed (multiple of 64).
//  mode K: every segment has M x N outputs at c + s * c_sstride (ldc); its
//          k range is [kpad_off[s], kpad_off[s + 1]) of A ([M][*], lda) and
//          B ([N][*], ldb), both TY.
struct BGemmArgs {
  int mode;  // 0 = R, 1 = K
  int S;     // segments
  const int* seg_start;
  const int* seg_count;
  const int* kpad_off;
  const void* a;
  long lda;
  int a_dtype;
  const int* a_map;
  int a_div;
  const void* b;
  long ldb;
  long b_sstride;
  float* c;
  long ldc;
  long c_sstride;
  int M, N, K;     // M: mode K only; N: columns computed; K: mode R only
  int n_store;     // columns stored (<= N)
  int max_rows;    // mode R: upper bound of the summed row count (grid size)
  int swf;         // launch_fgemm only (see there)
  const int* tile_off;  // mode R, optional: [S+1] prefix of the segments' row
                        // tile counts at the kernel's tile height
};
hipError_t launch_bgemm(int ty, const BGemmArgs& a, hipStream_t st);

// Wide variant (N a multiple of 64): B is fragment-major, [N/32][Kd/16][64
// lanes] fragments in the tile engine's permuted k order (Kd = K in mode R,
// ldb = the padded total in mode K, k-step offset kpad_off[s] / 16), and A
// rows are staged through LDS; 128 x 256 tiles of C (64 x 256 in fp32).
// swf > 0: B is the SwiGLU-interleaved first projection, whose fragment
// column n is C column ((n / 32) & 1) swf + (n / 64) 32 + n % 32.
hipError_t launch_fgemm(int ty, const BGemmArgs& a, hipStream_t st);

// Thin products over segments of rows, transposed on the fly:
//   C[s][m][n] = sum over rows p of segment s of A(p, m) B(p, n), n < N <= 32,
// A rows a_map ? a_map[p] / a_div : p of a row-major matrix (type a_dtype,
// ld lda, columns from a_c0), B rows p of a row-major fp32 matrix (ldb,
// columns from b_c0).  Column n of C goes to c_lo (n < 16) or c_hi (n - 16)
// at [s * c_sstride + m * ldc + n % 16] when n % 16 < n_store.  Each segment
// is summed in row order by one workgroup (no atomics).
struct TGemmArgs {
  int S;
  const int* seg_start;
  const int* seg_count;
  const void* a;
  int a_dtype;
  long lda;
  int a_c0;
  const int* a_map;
  int a_div;
  const float* b;
  long ldb;
  int b_c0;
  int N, M;
  float* c_lo;
  float* c_hi;
  long c_sstride;
  int ldc, n_store;
};
hipError_t launch_tgemm(int ty, const TGemmArgs& a, hipStream_t st);

// Fragment-major copy of row-major [G][N][Kd] (type TY, group strides in
// elements), rows padded with zeros to a multiple of 64.
hipError_t launch_plain_to_frag(int ty, const void* in, int G, long g_stride_in, int N, int Kd, void* out,
                                long g_stride_out, hipStream_t st);

// out[c][kpad_off[s] + r] = TY(in(row(s, r), c0 + c)) for r < count[s], zero
// for count[s] <= r < padded length; in rows are in_map ? in_map[start[s] + r]
// / in_div : start[s] + r of a row-major [*][ld_in] matrix of in_dtype.
struct TransArgs {
  int S;
  const int* start;
  const int* count;
  const int* kpad_off;
  const void* in;
  int in_dtype;
  long ld_in;
  int c0, ncols;
  const int* in_map;
  int in_div;
  void* out;
  long ld_out;
  int max_cols_k;  // upper bound of kpad_off[S] (grid size)
  int frag;        // 1: write the fragment-major image of out ([rows/32][ld_out/16][64]
                   // fragments, rows padded with zeros to a multiple of 32)
};
hipError_t launch_gather_t(int ty, const TransArgs& a, hipStream_t st);

// tile_off[0] = 0, tile_off[s + 1] = tile_off[s] + ceil(count[s] / rows)
hipError_t launch_tile_scan(const int* count, int S, int rows, int* tile_off, hipStream_t st);
// row tile height of launch_fgemm for MFMA type ty (launch_bgemm: 128)
int fgemm_rows(int ty);

// kpad_off[0] = 0, kpad_off[s + 1] = kpad_off[s] + roundup(count[s], 64)
hipError_t launch_pad_scan(const int* count, int S, int* kpad_off, hipStream_t st);

// Plain (row-major) copy of a fragment-major matrix frag(N, Kd), permuted
// k order: out[ (transpose ? k : nmap(n)) * ld_out + (transpose ? nmap(n) : k) ]
// with nmap the SwiGLU gate/up de-interleave when swiglu_f > 0 (fragment
// column n holds projection (n / 32) & 1, column (n / 64) * 32 + n % 32).
hipError_t launch_frag_to_plain(int ty, const void* frag, int G, long g_stride_in, int N, int Kd, int swiglu_f,
                                bool transpose, void* out, long g_stride_out, long ld_out, hipStream_t st);

// Per expert-list position p (expert-major, tokens ascending inside an
// expert): the assignment t*k + slot, its group row, gate weight and the
// row's u and e vectors of that expert, gathered once; apos inverts arow.
struct AssignArgs {
  int Na, E, K, k, ke, Pin, r;
  const int* perm;     // [Na] token of position p
  const int* offsets;  // [E+1]
  const int* idx;      // [T][k]
  const float* w;      // [T][k]
  const int* grow;     // [T kg] (t, group rank) -> group row
  const float* U;      // [R][NU]: u of expert j, projection p at (j Pin + p) 16
  int NU;
  const float* Eb;     // [R][NE]: e of expert j at j 16
  int NE;
  int* arow;           // [Na]  t*k + slot
  int* apos;           // [T k] position of (t, slot)
  int* prow;           // [Na]  group row
  float* pw;           // [Na]  gate weight
  float* ua;           // [Na][64]  u_gate | u_up | zeros (r > 0)
  float* ea;           // [Na][16]  (r > 0)
};
hipError_t launch_gather_assign(const AssignArgs& a, hipStream_t st);

// Activation backward over tiles of 64 positions of one expert, column
// split blockIdx.y of NS: z = Z + u B1^T, dh = w (D + e A2^T), h = act(z),
// dz = act'(z) dh.  Writes dz [Na][Pin f] and w h [Na][f] (type TY) and,
// per position and split, the column sums (dz_gate B1_gate, dz_up B1_up,
// h A2, <D, h>) to part[s][p][0..49).
struct ActArgs {
  int Na, E, f, Pin, act, r, NS;
  const int* offsets;
  const int* counts;
  const int* kpad;     // [E+1] 64-padded prefix of counts (tile walk)
  const int* prow;
  const float* pw;
  const float* ua;
  const float* ea;
  const float* Zb;     // [R][Pin f]
  const float* D;      // [R][f]
  const float* B1p;    // [E][Pin][f][16]
  const float* Adp;    // [E][f][16]
  void* dz;
  void* wh;
  float* part;         // [NS][Na][64]
};
constexpr int ACT_PART = 64;
hipError_t launch_act(int ty, const ActArgs& a, hipStream_t st);

// The same for layers without residuals (a.r == 0; part, NS, ua, ea, B1p
// and Adp unused): one wavefront per position along the columns, writing
// dz, w h and dw[arow[p]] = <D, h> directly.
hipError_t launch_act_plain(int ty, const ActArgs& a, const int* arow, float* dw, hipStream_t st);

// Sums the NS partials of each position in split order: q[p][0..Pin 16)
// (q[p][Pin 16..64) = 0), wu2[p] = w_p (h A2), dw[arow[p]] = <D, h> + <e, h A2>.
hipError_t launch_act_finish(const float* part, int NS, int Na, int Pin, int r, const float* pw, const float* ea,
                             const int* arow, float* q, float* wu2, float* dw, hipStream_t st);

// dZbar[row] = sum over the row's ke assignments (slot order) of dz and
// hbar[row] likewise of w h; fp32 sums stored in type TY.
hipError_t launch_row_sums(int ty, const void* dz, const void* wh, const int* garow, const int* apos, int R, int kg,
                           int ke, int k, int f, int Pin, void* dZbar, void* hbar, hipStream_t st);

// Per-token router backward and dX assembly: dX = sum over the token's
// group rows of dXb + sum over its assignments of dXr + router terms.
struct TokArgs {
  int T, d, G, K, kg, ke, k, r;
  int cols;             // dX columns per workgroup (a multiple of 4)
  const int* idx;
  const int* gidx;
  const float* w;
  const float* dw;      // [T k]
  const int* grow;      // [T kg]
  const int* apos;      // [T k]
  const float* dXb;     // [R][d]
  const float* dXr;     // [Na][d] (r > 0)
  const float* Wr;      // router matrix [d/16][NCp][16]
  int NCp;
  float* ds;            // [T kg][1 + K] group / expert logit gradients
  void* dX;
  int x_dtype;
};
hipError_t launch_tok(const TokArgs& a, hipStream_t st);

// row -> t*kg + rank map inverse: grow[t*kg + rank] = row
hipError_t launch_invert_rows(const int* garow, int R, int* grow, hipStream_t st);

// A1T[e][n][p*16 + rho] = Atp[e][p][n][rho] in type TY, zero for k >= Pin*16
// (the k-major operand of dXr = q A1^T, K = 64).
hipError_t launch_a1t(int ty, const float* Atp, int E, int Pin, int d, void* A1T, hipStream_t st);

hipError_t launch_zero_f(float* p, long n, hipStream_t st);
// out[s * ld_out + c] = sum over the rows of segment s of in[map(row)][c], c < ncols
hipError_t launch_seg_colsum(const float* in, long ld_in, int ncols, const int* start, const int* count,
                             const int* in_map, int S, float* out, long ld_out, hipStream_t st);
// plain k-major copies of the residual factors for the backward GEMMs:
// out[g][(j * P + p) * 16 + rho][k] = src[(g K + j)][p][k][rho] (TY), padded rows zero
hipError_t launch_stack_factors(int ty, const float* src, int G, int K, int P, int n, int rows_out, void* out,
                                hipStream_t st);

}  // namespace cefn
