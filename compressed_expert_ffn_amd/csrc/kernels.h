// Internal interface between the host layer (api.hip) and the kernels.
//
// Device weight layouts (built by api.hip with pack.h at create time):
//
//  "fragment-major" for a matrix with N columns and depth Kd (the MFMA k):
//     [N/32][Kd/16][64 lanes][8]: fragment (n/32, ks), lane (n%32) + 32h,
//     slot e holds k = frag_k(ks, h, e) -- one 16-deep k-step of a 32-column
//     block is 64 x 8 contiguous elements, one coalesced 16-byte load per
//     lane.  Matrices whose depth is a multiple of 64 use the permuted k
//     order of tile.h (lane half h covers 32 consecutive k of each 64-deep
//     block); the 16-deep residual steps (B1) use the plain order.
//  INT4 factors use the same order with 8 nibbles (q + 8, element e in bits
//  4e..4e+3) in one 32-bit word per lane, plus fp16 scales.
//
//  W1   [G] x frag(N = P_in*f, Kd = d)  input projections of the base; for
//       SwiGLU the N order interleaves 32-column blocks gate, up, gate, up...
//  W2   [G] x frag(N = d, Kd = f)       output projection of the base
//  At   [G] x frag(N = NU, Kd = d)      column (j*P_in + p)*RPAD + rho holds
//       A_{p, gK+j}[:, rho] (zero for rho >= r and for padding columns);
//       INT4 scales [G][NU/32][d/32][32]
//  B1   [E][P_in] x frag(N = f, Kd = RPAD)  B_p^T; INT4 scales [E][P_in][f/32][RPAD]
//  Ad   [E][f/32][2][64][8]  A_down as the MFMA operand of the fused
//       h . A_down product: lane rho + 32h, slot e of step s holds row
//       fb*32 + ad_row(s, h, e) (pack.h); INT4 scales [E][f/32][RPAD]
//  Bd   [G] x frag(N = d, Kd = NV)  row j*RPAD + rho of the k axis holds
//       B_{down, gK+j}[:, rho]; INT4 scales [E][d/32][RPAD]
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cefn {

struct RouteArgs {
  const void* X;
  int T, d, G, K, kg, ke, k, E;
  const uint16_t* Wb;  // 16-bit activations: the same matrix as three bf16 parts
                       // [3][d/16][NCp][16], W = part 0 + part 1 + part 2 to
                       // within 2^-24 relative (split on the host)
  const float* Wr;     // router matrix [d/16][NCp][16]: column c < G is W_grp[:, c],
                       // column G + g*K + j is W_exp[g][:, j], the rest zero;
                       // element (k, c) at ((k/16) * NCp + c) * 16 + k % 16
  int NCp;             // score columns, G (+ G*K when K > 1), padded to 32
  float* L;            // scores [nsplit][T][NCp] (partial sums over k splits)
  int nsplit;          // k splits of the score GEMM (router_splits)
  const float* gbias;  // [G] or null
  const float* ebias;  // [E] or null
  int* idx;            // [T][k]
  float* w;            // [T][k]
  int* gidx;           // [T][kg]
  int* ccount;         // [chunks of T*k][E], zero on entry
  int* cgcount;        // [chunks of T*kg][G], zero on entry
  int count_experts;   // 0: skip the expert-level counters (group lists only)
};

struct ScatterArgs {
  int T, k, kg, E, G;
  const int* idx;
  const int* gidx;
  const int* ccount;
  const int* cgcount;
  int nch_e, nch_g;
  int* counts;    // [E]
  int* offsets;   // [E+1]
  int* perm;      // [T*k] token ids, or null
  int* gcounts;   // [G]
  int* goffsets;  // [G+1]
  int* gperm;     // [T*kg] token ids, or null
  int* garow;     // [T*kg] group-list position -> t*kg + group rank
  int do_experts; // 0: build the group lists only
};

// Rows of each group list reordered by the expert set of the row (forward
// pass only; the internal row map, not the routing outputs): one
// workgroup per group, counting sort on the set folded to 8 bits.
struct GroupSortArgs {
  const int* garow_in;   // [T*kg] group-list position -> t*kg + group rank
  int* garow_out;        // [T*kg] the same rows, sorted inside each group
  const int* goffsets;   // [G+1]
  const int* idx;        // [T*k]
  int G, K, kg, ke, k;
};

// Common to the three grouped GEMMs.  Rows are group-list positions
// (goffsets[g] <= row < goffsets[g+1]); a tile is (group, BM rows) x (256 cols).
struct GemmArgs {
  const int* gcounts;
  const int* goffsets;
  int G, K, kg, ke, k;
  int resid;            // RS_*
  int act;              // ACT_*
  // activations
  const void* X;        // [T][d] x dtype (U, G1)
  int d, f;
  const int* garow;     // [T*kg]
  const int* idx;       // [T][k]
  const float* w;       // [T][k]
  // weights (fragment-major, per group unless noted)
  const void* Bw;       // W1 (G1), W2 (G2), At (U)
  long bw_gstride;      // elements (or 32-bit words for INT4 At) per group
  const uint16_t* bw_scale;  // INT4 scales of At
  long bws_gstride;
  const void* B1;       // G1 residual B (per expert)
  const uint16_t* b1_scale;
  const void* Ad;       // G1 A_down (per expert)
  const uint16_t* ad_scale;
  const void* Bd;       // G2 residual tail (per group)
  long bd_gstride;
  const uint16_t* bd_scale;
  // workspace
  void* U;              // [rows][NU] MFMA type
  int NU;
  void* V;              // [rows][NV] MFMA type (G2 tail input)
  int NV;
  float* Vp;            // [G1 column tiles][vp_rows][ke][16] partials of V
  long vp_rows;
  void* H;              // [rows][f] MFMA type
  float* ypart;         // [ksplit][T*kg][d] fp32 partials (kg > 1 or ksplit > 1)
  void* Y;              // [T][d] x dtype (kg == 1 and one k split)
  int ksplit;           // G2: k splits of the base part (partials in ypart)
  long rows_total;      // T * kg
  int* zero_ptr;        // cleared by the output GEMM's first block
  int zero_n;
  int rows_sorted;      // G1: group lists already ordered by expert set (tiles keep that order)
  const int* gslot;     // weights of group g sit at slot gslot[g] of the weight arrays (null: g)
  // G2 last-round split (tail_slots > 0; one k split):
  // resident workgroups per round, most pieces per tile, room in tailpart
  // for this many partial tiles of BM x 256 floats
  int tail_slots, tail_smax, tail_max_pieces;
  float* tailpart;
};

struct VReduceArgs {
  const float* Vp;
  void* V;  // MFMA type
  const int* garow;
  const int* gidx;
  const int* idx;
  long vp_rows;
  int rows, ntiles, NV, K, kg, ke, k;
};

struct CombineArgs {
  const float* ypart;
  void* Y;
  int T, d, kg, ksplit;
};

// G2K: G2 with the k split inside a workgroup.  G1K: G1 with 32-row x
// 64-column tiles and d split over the four wavefronts (few rows per group;
// bm = 32, ntiles counted for 64 columns); G1K2: 32-row x 128-column tiles,
// d in two halves, each over two wavefronts of 64 columns (ntiles counted
// for 128 columns).  UT: U on the tile engine (BM-row x 256-column tiles;
// many rows).
enum GemmKind { GK_U = 0, GK_G1 = 1, GK_G2 = 2, GK_G2K = 3, GK_G1K = 4, GK_UT = 5, GK_G1K2 = 6 };

// most k splits of the router score GEMM (the selection sums that many
// partial score sets)
constexpr int kMaxRouterSplits = 16;
hipError_t launch_router(int x_dtype, const RouteArgs& a, hipStream_t st);
int router_splits(int T, int d, int NCp);
// max_rows: an upper bound on any group's row count (sizes the key cache)
// bf16 X -> fp16 copy (n elements, a multiple of 8)
hipError_t launch_cvt_x(const void* X, void* X16, long n, hipStream_t st);
hipError_t launch_group_sort(const GroupSortArgs& a, int max_rows, hipStream_t st);
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t st);
size_t scatter_lds_bytes(int E, int G);
hipError_t launch_zero(int* p, int n, hipStream_t st);

// bm (32, 64, 128, 256; fp32: 32, 64) token rows x 256 columns per tile;
// max_mtiles: upper bound of sum_g ceil(M_g / bm); ntiles: column tiles of
// 256; splits: k splits (G2 only, 1 otherwise).
hipError_t launch_gemm(int kind, int x_dtype, int mma_dtype, int bm, const GemmArgs& a, int max_mtiles,
                       int ntiles, int splits, hipStream_t st);
// LDS bytes of one tile (K experts per group, ke chosen per group)
size_t gemm_lds(int kind, int mma_dtype, int bm, int K, int ke);

// LDS layout of an input-projection workgroup of bm rows (the kernel and
// gemm_lds both use it).  Region A holds the token stages during the main
// loop, then the V slices (one per wavefront: 32 rows x (ke*RPAD + 1)
// floats), two sets of them when the whole layout still fits two
// workgroups per compute unit (80 KB; 160 KB at 256 rows), so consecutive
// token blocks alternate sets and need one barrier each; the k-split form
// (ks) keeps one set and also puts its four partial tiles there.  Then
// gate weights [bm][K] floats, slots [bm][K] int8, the token blocks' expert
// bit sets, the row order and key histogram [bm + 260] ints, and (ks) the h
// sums [4][2][16][64] floats.
struct G1Lds {
  size_t vbytes;  // one set of V slices
  bool vdb;       // two sets
  size_t abytes;  // region A
  size_t total;
};
__host__ __device__ inline G1Lds g1_lds(bool ks, int mma_dtype, int bm, int K, int ke) {
  auto al16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
  const size_t fb = mma_dtype == 0 ? 32 : 16;  // fragment bytes (fp32, dtype 0: 32)
  const size_t tbytes = 2 * (size_t)(bm / 32) * 4 * 64 * fb;
  G1Lds L;
  L.vbytes = (size_t)4 * 32 * (ke * 16 + 1) * sizeof(float);
  const size_t rest = sizeof(float) * bm * K + al16((size_t)bm * K) + sizeof(uint32_t) * 2 * (bm / 32) +
                      sizeof(int) * ((size_t)bm + 260) + (ks ? (size_t)4 * 2 * 16 * 64 * sizeof(float) : 0) + 64;
  const size_t a2 = al16(tbytes > 2 * L.vbytes ? tbytes : 2 * L.vbytes);
  L.vdb = !ks && a2 + rest <= (bm >= 256 ? 160 * 1024 : 80 * 1024);
  size_t a = tbytes > L.vbytes ? tbytes : L.vbytes;
  if (ks && a < (size_t)4 * 2 * 16 * 64 * sizeof(float)) a = (size_t)4 * 2 * 16 * 64 * sizeof(float);
  L.abytes = L.vdb ? a2 : al16(a);
  L.total = L.abytes + rest;
  return L;
}
hipError_t launch_vreduce(int mma_dtype, const VReduceArgs& a, hipStream_t st);
hipError_t launch_combine(int x_dtype, const CombineArgs& a, hipStream_t st);
// after a G2 launch with tail_slots > 0 (same arguments and tile height)
hipError_t launch_tailfix(int x_dtype, int bm, const GemmArgs& a, hipStream_t st);

// Device-side decode of stored residual factors (test export).
hipError_t launch_debug_decode(int mma_dtype, int resid, int kind, const void* src,
                               const uint16_t* scales, long base, long sbase, int n, int r,
                               int aux0, int aux1, float* out, int ldo, hipStream_t st);

}  // namespace cefn
