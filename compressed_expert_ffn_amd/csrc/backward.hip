// moe_backward: the C ABI of the backward pass (kernels in train.hip).
#include <algorithm>
#include <memory>

#include "api_internal.h"

using namespace cefn;
using namespace cefn_api;

// ---------------------------------------------------------- backward ----
// Plain k-major weight copies and the workspace of moe_backward, built on
// its first call from the device layouts (no host copy of the weights is
// kept).  U, E and the residual factors are kept as float32 for the
// elementwise steps; GEMM operands are in the MFMA type.
struct BwdState {
  // fragment-major (tile engine layout) B operands: W1^T [d][Pin f], W2^T
  // [f][d], stacked A1 [NUp][d] and B2 [NEp][d] per group, A1 [d][64] per expert
  void *W1F = nullptr, *W2F = nullptr, *AtF = nullptr, *BdF = nullptr, *A1F = nullptr;
  float *Atp = nullptr, *B1p = nullptr, *Adp = nullptr;
  int NUb = 0, NEb = 0, NUp = 0, NEp = 0;  // stacked factor rows, and rounded up to 64
  long Kg = 0, KgF = 0, part_cap = 0;
  int *counts = nullptr, *offsets = nullptr, *perm = nullptr, *arow = nullptr, *apos = nullptr, *prow = nullptr;
  int *grow = nullptr, *kpad_g = nullptr, *kpad_e = nullptr, *toff_g = nullptr, *toff_e = nullptr;
  float *Zb = nullptr, *U = nullptr, *D = nullptr, *Eb = nullptr, *pw = nullptr, *part = nullptr;
  float *q = nullptr, *wu2 = nullptr, *dw = nullptr, *ua = nullptr, *ea = nullptr, *dXb = nullptr, *dXr = nullptr;
  float *ds = nullptr;
  void *dz = nullptr, *wh = nullptr, *dZbar = nullptr, *hbar = nullptr;
  void *XTg = nullptr, *dZT = nullptr, *hbT = nullptr, *dYTg = nullptr, *dsdeT = nullptr;
};

namespace cefn_api {

void delete_bwd(moe_handle* h) {
  delete h->bwd;
  h->bwd = nullptr;
}

}  // namespace cefn_api

// ---- backward pass -------------------------------------------------------
namespace {

// Build the backward layouts and workspace (first moe_backward call).
int prepare_backward(moe_handle* h) {
  if (h->bwd) return MOE_OK;
  const moe_config& c = h->cfg;
  std::unique_ptr<BwdState> B(new BwdState());
  const int G = c.G, K = c.K, E = h->E, Pin = h->P_in, d = c.d, f = c.f, r = c.r, ty = h->mma;
  const size_t es = elem_bytes(ty);
  const long T = c.T_max, R = T * c.top_groups, Na = T * h->k;
  hipStream_t st = nullptr;
  hipError_t e;
  char* tmp = nullptr;
  auto alloc_bytes = [&](void** p, size_t bytes) -> int {
    char* q = nullptr;
    TRY(dalloc(h, &q, bytes + 256));
    *p = q;
    return MOE_OK;
  };
  auto alloc_f = [&](float** p, size_t n) { return dalloc(h, p, n + 64); };
  auto alloc_i = [&](int** p, size_t n) { return dalloc(h, p, n + 64); };
  // plain copies go through one scratch buffer into the fragment-major images
  size_t tmp_bytes = (size_t)G * Pin * f * d * es;
  if (r > 0) tmp_bytes = std::max({tmp_bytes, (size_t)E * d * 64 * es, (size_t)G * K * Pin * 16 * d * es});
  struct Tmp {
    char* p = nullptr;
    ~Tmp() {
      if (p) (void)hipFree(p);
    }
  } scratch;
  if (hipMalloc(&scratch.p, tmp_bytes) != hipSuccess) return fail(MOE_ERR_OOM, "backward set-up scratch");
  tmp = scratch.p;
  TRY(alloc_bytes(&B->W1F, (size_t)G * Pin * f * d * es));
  TRY(alloc_bytes(&B->W2F, (size_t)G * f * d * es));
  const int swf = Pin > 1 ? f : 0;
  e = launch_frag_to_plain(ty, h->W1, G, h->w1_gs, Pin * f, d, swf, true, tmp, (long)Pin * f * d, (long)Pin * f, st);
  if (e == hipSuccess) e = launch_plain_to_frag(ty, tmp, G, (long)Pin * f * d, d, Pin * f, B->W1F, (long)Pin * f * d, st);
  if (e == hipSuccess) e = launch_frag_to_plain(ty, h->W2, G, h->w2_gs, d, f, 0, true, tmp, (long)f * d, d, st);
  if (e == hipSuccess) e = launch_plain_to_frag(ty, tmp, G, (long)f * d, f, d, B->W2F, (long)f * d, st);
  if (e != hipSuccess) return hip_fail(h, e, "backward weight repack");
  if (r > 0) {
    B->NUb = K * Pin * 16;
    B->NEb = K * 16;
    B->NUp = (B->NUb + 63) / 64 * 64;
    B->NEp = (B->NEb + 63) / 64 * 64;
    TRY(alloc_f(&B->Atp, (size_t)E * Pin * d * 16));
    TRY(alloc_f(&B->B1p, (size_t)E * Pin * f * 16));
    TRY(alloc_f(&B->Adp, (size_t)E * f * 16));
    float* Bdp = nullptr;
    TRY(alloc_f(&Bdp, (size_t)E * d * 16));
    e = launch_zero_f(B->Atp, (long)E * Pin * d * 16, st);
    if (e == hipSuccess) e = launch_zero_f(B->B1p, (long)E * Pin * f * 16, st);
    if (e == hipSuccess) e = launch_zero_f(B->Adp, (long)E * f * 16, st);
    if (e == hipSuccess) e = launch_zero_f(Bdp, (long)E * d * 16, st);
    for (int i = 0; i < E && e == hipSuccess; ++i)
      for (int p = 0; p < h->P && e == hipSuccess; ++p)
        for (int which = 0; which < 2 && e == hipSuccess; ++which) {
          const FactorLoc L = locate_factor(h, p, which, i);
          float* out;
          if (p < Pin) out = which == 0 ? B->Atp + ((size_t)i * Pin + p) * d * 16 : B->B1p + ((size_t)i * Pin + p) * f * 16;
          else out = which == 0 ? B->Adp + (size_t)i * f * 16 : Bdp + (size_t)i * d * 16;
          e = launch_debug_decode(ty, c.resid, L.kind, L.src, L.sc, L.base, L.sbase, L.n, r, L.aux0, L.aux1, out, 16, st);
        }
    if (e != hipSuccess) return hip_fail(h, e, "backward factor decode");
    TRY(alloc_bytes(&B->AtF, (size_t)G * B->NUp * d * es));
    TRY(alloc_bytes(&B->BdF, (size_t)G * B->NEp * d * es));
    TRY(alloc_bytes(&B->A1F, (size_t)E * d * 64 * es));
    e = launch_stack_factors(ty, B->Atp, G, K, Pin, d, B->NUb, tmp, st);
    if (e == hipSuccess) e = launch_plain_to_frag(ty, tmp, G, (long)B->NUb * d, B->NUb, d, B->AtF, (long)B->NUp * d, st);
    if (e == hipSuccess) e = launch_stack_factors(ty, Bdp, G, K, 1, d, B->NEb, tmp, st);
    if (e == hipSuccess) e = launch_plain_to_frag(ty, tmp, G, (long)B->NEb * d, B->NEb, d, B->BdF, (long)B->NEp * d, st);
    if (e == hipSuccess) e = launch_a1t(ty, B->Atp, E, Pin, d, tmp, st);
    if (e == hipSuccess) e = launch_plain_to_frag(ty, tmp, E, (long)d * 64, d, 64, B->A1F, (long)d * 64, st);
    if (e != hipSuccess) return hip_fail(h, e, "backward factor stacking");
  }
  if (hipStreamSynchronize(st) != hipSuccess) return fail(MOE_ERR_HIP, "backward weight repack failed");
  // workspace for T_max tokens
  // (multiples of 64, so every transposed row starts 128-byte aligned)
  B->Kg = (R + 64L * G + 63) / 64 * 64;
  B->KgF = B->Kg;
  // act_splits(Na, E, f) * Na <= 1024 * 64 + Na for every Na
  B->part_cap = 1024L * 64 + Na;
  TRY(alloc_i(&B->counts, E));
  TRY(alloc_i(&B->offsets, E + 1));
  TRY(alloc_i(&B->perm, Na));
  TRY(alloc_i(&B->arow, Na));
  TRY(alloc_i(&B->apos, Na));
  TRY(alloc_i(&B->prow, Na));
  TRY(alloc_i(&B->grow, R));
  TRY(alloc_i(&B->kpad_g, G + 1));
  TRY(alloc_i(&B->kpad_e, E + 1));
  TRY(alloc_i(&B->toff_g, G + 1));
  TRY(alloc_i(&B->toff_e, E + 1));
  TRY(alloc_f(&B->pw, (size_t)Na));
  TRY(alloc_f(&B->part, (size_t)B->part_cap * ACT_PART));
  TRY(alloc_f(&B->Zb, (size_t)R * Pin * f));
  TRY(alloc_f(&B->D, (size_t)R * f));
  if (K > 1) {  // (one expert per group: dz and w h serve as dZbar and hbar)
    TRY(alloc_bytes(&B->dZbar, (size_t)R * Pin * f * es));
    TRY(alloc_bytes(&B->hbar, (size_t)R * f * es));
  }
  TRY(alloc_f(&B->dw, (size_t)Na));
  TRY(alloc_f(&B->dXb, (size_t)R * d));
  TRY(alloc_f(&B->ds, (size_t)R * (1 + K)));
  TRY(alloc_bytes(&B->dz, (size_t)Na * Pin * f * es));
  TRY(alloc_bytes(&B->wh, (size_t)Na * f * es));
  TRY(alloc_bytes(&B->XTg, (size_t)d * B->Kg * es));
  TRY(alloc_bytes(&B->dZT, (size_t)Pin * f * B->KgF * es));
  TRY(alloc_bytes(&B->hbT, (size_t)f * B->Kg * es));
  TRY(alloc_bytes(&B->dYTg, (size_t)d * B->KgF * es));
  TRY(alloc_bytes(&B->dsdeT, (size_t)(1 + K) * B->Kg * es));
  if (r > 0) {
    TRY(alloc_f(&B->U, (size_t)R * B->NUb));
    TRY(alloc_f(&B->Eb, (size_t)R * B->NEb));
    TRY(alloc_f(&B->q, (size_t)Na * 64));
    TRY(alloc_f(&B->wu2, (size_t)Na * 16));
    TRY(alloc_f(&B->ua, (size_t)Na * 64));
    TRY(alloc_f(&B->ea, (size_t)Na * 16));
    TRY(alloc_f(&B->dXr, (size_t)Na * d));
  }
  (void)tmp;
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_ERR_HIP, "backward set-up failed");
  h->bwd = B.release();
  return MOE_OK;
}

// Column splits of the activation backward: enough workgroups for the chip
// (about 1024) when there are few 64-position tiles.
int act_splits(long Na, int E, int f) {
  // tiles: full ones plus about half of the experts' partial ones
  const long tiles = std::max(1L, (Na + 63) / 64 + std::min<long>(E, Na) / 2);
  long ns = (1024 + tiles - 1) / tiles;
  ns = std::min<long>(ns, f / 64);
  return (int)std::max(1L, ns);
}

BGemmArgs rgemm(const Workspace& ws, const int* gcounts, const int* goffsets, int G, long R, const void* a, long lda,
                int a_dtype, const int* a_map, int a_div, const void* b, long b_sstride, int N, int K, float* c,
                long ldc) {
  (void)ws;
  BGemmArgs g{};
  g.mode = 0;
  g.S = G;
  g.seg_start = goffsets;
  g.seg_count = gcounts;
  g.a = a;
  g.lda = lda;
  g.a_dtype = a_dtype;
  g.a_map = a_map;
  g.a_div = a_div;
  g.b = b;
  g.ldb = K;
  g.b_sstride = b_sstride;
  g.c = c;
  g.ldc = ldc;
  g.N = N;
  g.K = K;
  g.n_store = N;
  g.max_rows = (int)R;
  return g;
}

// the wide kernel's N (a multiple of 64) over a B padded to that many rows
BGemmArgs widen(BGemmArgs g, int n_padded) {
  g.N = n_padded;
  return g;
}

BGemmArgs kgemm(int S, const int* kpad, int ty, const void* a, long lda, const void* b, long ldb, int M, int N,
                float* c, long c_sstride, long ldc, int n_store) {
  BGemmArgs g{};
  g.mode = 1;
  g.S = S;
  g.kpad_off = kpad;
  g.a = a;
  g.lda = lda;
  g.a_dtype = ty;
  g.b = b;
  g.ldb = ldb;
  g.c = c;
  g.c_sstride = c_sstride;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.n_store = n_store;
  return g;
}

TransArgs tgather(int S, const int* start, const int* count, const int* kpad, const void* in, int in_dtype, long ld_in,
                  int c0, int ncols, const int* map, int div, void* out, long ld_out, long max_k, int frag = 0) {
  TransArgs t{};
  t.frag = frag;
  t.S = S;
  t.start = start;
  t.count = count;
  t.kpad_off = kpad;
  t.in = in;
  t.in_dtype = in_dtype;
  t.ld_in = ld_in;
  t.c0 = c0;
  t.ncols = ncols;
  t.in_map = map;
  t.in_div = div;
  t.out = out;
  t.ld_out = ld_out;
  t.max_cols_k = (int)max_k;
  return t;
}

}  // namespace

extern "C" {

int moe_backward(moe_handle* h, const void* X, int32_t T, const void* dY, void* dX, const moe_grads* gr,
                 void* stream) {
  if (!h || !gr) return fail(MOE_ERR_INVALID_ARG, "null handle or gradients");
  const moe_config& c = h->cfg;
  if (T < 0 || T > c.T_max) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, T_max=%d]", T, c.T_max);
  if (T > 0 && (!X || !dY || !dX)) return fail(MOE_ERR_INVALID_ARG, "null X, dY or dX");
  const int G = c.G, K = c.K, E = h->E, Pin = h->P_in, P = h->P, d = c.d, f = c.f, r = c.r, ty = h->mma;
  const int kg = c.top_groups, k = h->k;
  for (int p = 0; p < P; ++p)
    if (!gr->dbase[p] || (r > 0 && (!gr->dA[p] || !gr->dB[p])))
      return fail(MOE_ERR_INVALID_ARG, "gradient buffer of projection %d is null", p);
  if (!gr->dW_grp) return fail(MOE_ERR_INVALID_ARG, "dW_grp is null");
  if (h->off) return fail(MOE_ERR_UNSUPPORTED, "the handle's groups are offloaded");
  TRY(prepare_backward(h));
  BwdState* B = h->bwd;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t x) { if (e == hipSuccess) e = x; };
  if (T == 0) {
    for (int p = 0; p < P; ++p) {
      int di, dn;
      dims(c, p, di, dn);
      ok(launch_zero_f(gr->dbase[p], (long)G * di * dn, st));
      if (r > 0) {
        ok(launch_zero_f(gr->dA[p], (long)E * di * r, st));
        ok(launch_zero_f(gr->dB[p], (long)E * dn * r, st));
      }
    }
    ok(launch_zero_f(gr->dW_grp, (long)d * G, st));
    if (gr->dW_exp) ok(launch_zero_f(gr->dW_exp, (long)G * d * K, st));
    if (gr->d_group_bias) ok(launch_zero_f(gr->d_group_bias, G, st));
    if (gr->d_expert_bias) ok(launch_zero_f(gr->d_expert_bias, E, st));
    return e == hipSuccess ? MOE_OK : hip_fail(h, e, "backward (no tokens)");
  }
  // routing again (the forward pass's decisions), with the expert lists
  Prof pf{h, st, -1};
  RouteLive live{};
  moe_route_out ro{};
  ro.counts = B->counts;
  ro.offsets = B->offsets;
  ro.perm = B->perm;
  TRY(run_route(h, h->ws, X, T, &ro, true, st, pf, live));
  ok(launch_zero(h->ws.cc, h->ws.cc_n, st));
  const long R = (long)T * kg, Na = (long)T * k;
  const int* garow = h->ws.garow;
  const size_t es = elem_bytes(ty);
  // forward intermediates: Z = X W1_base per group row, U = X A1 stacked
  // row tiles of the wide GEMMs per group and per expert
  const int fm = fgemm_rows(ty);
  ok(launch_tile_scan(live.gcounts, G, fm, B->toff_g, st));
  ok(launch_tile_scan(B->counts, E, fm, B->toff_e, st));
  auto tg = [&](BGemmArgs g) {
    g.tile_off = g.S == E && g.seg_count == B->counts ? B->toff_e : B->toff_g;
    return g;
  };
  // (the forward pass's own fragment-major W1, SwiGLU-interleaved columns)
  {
    BGemmArgs g = rgemm(h->ws, live.gcounts, live.goffsets, G, R, X, d, c.x_dtype, garow, kg, h->W1, h->w1_gs,
                        Pin * f, d, B->Zb, (long)Pin * f);
    g.swf = Pin > 1 ? f : 0;
    ok(launch_fgemm(ty, tg(g), st));
  }
  if (r > 0)
    ok(launch_fgemm(ty, tg(widen(rgemm(h->ws, live.gcounts, live.goffsets, G, R, X, d, c.x_dtype, garow, kg, B->AtF,
                                       (long)B->NUp * d, B->NUb, d, B->U, B->NUb), B->NUp)), st));
  // D = dY W2_base^T, E = dY B2 stacked
  ok(launch_fgemm(ty, tg(rgemm(h->ws, live.gcounts, live.goffsets, G, R, dY, d, c.x_dtype, garow, kg, B->W2F,
                               (long)f * d, f, d, B->D, f)), st));
  if (r > 0)
    ok(launch_fgemm(ty, tg(widen(rgemm(h->ws, live.gcounts, live.goffsets, G, R, dY, d, c.x_dtype, garow, kg, B->BdF,
                                       (long)B->NEp * d, B->NEb, d, B->Eb, B->NEb), B->NEp)), st));
  // per expert-list position: assignment, row, weight, u and e
  const int ke = c.top_experts;
  ok(launch_invert_rows(garow, (int)R, B->grow, st));
  ok(launch_pad_scan(B->counts, E, B->kpad_e, st));
  {
    AssignArgs as{};
    as.Na = (int)Na;
    as.E = E;
    as.K = K;
    as.k = k;
    as.ke = ke;
    as.Pin = Pin;
    as.r = r;
    as.perm = B->perm;
    as.offsets = B->offsets;
    as.idx = live.idx;
    as.w = live.w;
    as.grow = B->grow;
    as.U = B->U;
    as.NU = B->NUb;
    as.Eb = B->Eb;
    as.NE = B->NEb;
    as.arow = B->arow;
    as.apos = B->apos;
    as.prow = B->prow;
    as.pw = B->pw;
    as.ua = B->ua;
    as.ea = B->ea;
    ok(launch_gather_assign(as, st));
  }
  // activation backward over expert tiles, then the per-position sums
  const int NS = act_splits(Na, E, f);
  if ((long)NS * Na > B->part_cap) return fail(MOE_ERR_UNSUPPORTED, "activation partials exceed their buffer");
  {
    ActArgs aa{};
    aa.Na = (int)Na;
    aa.E = E;
    aa.f = f;
    aa.Pin = Pin;
    aa.act = c.act == MOE_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU;
    aa.r = r;
    aa.NS = NS;
    aa.offsets = B->offsets;
    aa.counts = B->counts;
    aa.kpad = B->kpad_e;
    aa.prow = B->prow;
    aa.pw = B->pw;
    aa.ua = B->ua;
    aa.ea = B->ea;
    aa.Zb = B->Zb;
    aa.D = B->D;
    aa.B1p = B->B1p;
    aa.Adp = B->Adp;
    aa.dz = B->dz;
    aa.wh = B->wh;
    aa.part = B->part;
    if (r > 0) {
      ok(launch_act(ty, aa, st));
      ok(launch_act_finish(B->part, NS, (int)Na, Pin, r, B->pw, B->ea, B->arow, B->q, B->wu2, B->dw, st));
    } else {
      ok(launch_act_plain(ty, aa, B->arow, B->dw, st));
    }
  }
  // With one expert per group the expert lists are the group lists (the
  // same stable order), so position p is group row p: dZbar and hbar are dz
  // and w h themselves.
  void* dZbar = B->dZbar;
  void* hbar = B->hbar;
  if (K == 1) {
    dZbar = B->dz;
    hbar = B->wh;
  } else {
    ok(launch_row_sums(ty, B->dz, B->wh, garow, B->apos, (int)R, kg, ke, k, f, Pin, dZbar, hbar, st));
  }
  // dX: base part per group row, residual part per position, then per token
  ok(launch_fgemm(ty, tg(rgemm(h->ws, live.gcounts, live.goffsets, G, R, dZbar, (long)Pin * f, ty, nullptr, 1,
                               B->W1F, (long)Pin * f * d, d, Pin * f, B->dXb, d)), st));
  if (r > 0)
    ok(launch_fgemm(ty, tg(rgemm(h->ws, B->counts, B->offsets, E, Na, B->q, 64, MOE_F32, nullptr, 1, B->A1F,
                                 (long)d * 64, d, 64, B->dXr, d)), st));
  {
    TokArgs ta{};
    ta.T = T;
    ta.d = d;
    ta.G = G;
    ta.K = K;
    ta.kg = kg;
    ta.ke = ke;
    ta.k = k;
    ta.r = r;
    // few tokens: several workgroups per token
    ta.cols = T >= 1024 ? (d + 3) / 4 * 4 : 512;
    ta.idx = live.idx;
    ta.gidx = live.gidx;
    ta.w = live.w;
    ta.dw = B->dw;
    ta.grow = B->grow;
    ta.apos = B->apos;
    ta.dXb = B->dXb;
    ta.dXr = B->dXr;
    ta.Wr = h->Wr;
    ta.NCp = h->NCp;
    ta.ds = B->ds;
    ta.dX = dX;
    ta.x_dtype = c.x_dtype;
    ok(launch_tok(ta, st));
  }
  // weight gradients over each group's rows
  ok(launch_pad_scan(live.gcounts, G, B->kpad_g, st));
  const long Kg = B->Kg, KgF = B->KgF;
  ok(launch_gather_t(ty, tgather(G, live.goffsets, live.gcounts, B->kpad_g, X, c.x_dtype, d, 0, d, garow, kg, B->XTg,
                                 Kg, Kg), st));
  ok(launch_gather_t(ty, tgather(G, live.goffsets, live.gcounts, B->kpad_g, dZbar, ty, (long)Pin * f, 0,
                                 Pin * f, nullptr, 1, B->dZT, KgF, Kg, 1), st));
  ok(launch_gather_t(ty, tgather(G, live.goffsets, live.gcounts, B->kpad_g, hbar, ty, f, 0, f, nullptr, 1,
                                 B->hbT, Kg, Kg), st));
  ok(launch_gather_t(ty, tgather(G, live.goffsets, live.gcounts, B->kpad_g, dY, c.x_dtype, d, 0, d, garow, kg,
                                 B->dYTg, KgF, Kg, 1), st));
  ok(launch_gather_t(ty, tgather(G, live.goffsets, live.gcounts, B->kpad_g, B->ds, MOE_F32, 1 + K, 0, 1 + K, garow, 1,
                                 B->dsdeT, Kg, Kg), st));
  for (int p = 0; p < Pin; ++p)
    ok(launch_fgemm(ty, kgemm(G, B->kpad_g, ty, B->XTg, Kg, static_cast<char*>(B->dZT) + (size_t)p * f * KgF * es,
                              KgF, d, f, gr->dbase[p], (long)d * f, f, f), st));
  ok(launch_fgemm(ty, kgemm(G, B->kpad_g, ty, B->hbT, Kg, B->dYTg, KgF, f, d, gr->dbase[P - 1], (long)f * d, d, d),
                  st));
  // router weights and biases
  ok(launch_bgemm(ty, kgemm(G, B->kpad_g, ty, B->XTg, Kg, B->dsdeT, Kg, d, 1, gr->dW_grp, 1, G, 1), st));
  if (K > 1 && gr->dW_exp)
    ok(launch_bgemm(ty, kgemm(G, B->kpad_g, ty, B->XTg, Kg, static_cast<char*>(B->dsdeT) + (size_t)Kg * es, Kg, d, K,
                              gr->dW_exp, (long)d * K, K, K), st));
  else if (gr->dW_exp)
    ok(launch_zero_f(gr->dW_exp, (long)G * d * K, st));
  if (gr->d_group_bias)
    ok(launch_seg_colsum(B->ds, 1 + K, 1, live.goffsets, live.gcounts, garow, G, gr->d_group_bias, 1, st));
  if (gr->d_expert_bias) {
    if (K > 1)
      ok(launch_seg_colsum(B->ds + 1, 1 + K, K, live.goffsets, live.gcounts, garow, G, gr->d_expert_bias, K, st));
    else
      ok(launch_zero_f(gr->d_expert_bias, E, st));
  }
  // residual factor gradients over each expert's assignments (position
  // order), the row operands transposed on the fly
  if (r > 0) {
    auto tg = [&](const void* A, int adt, long lda, int ac0, const int* amap, int adiv, const float* Bm, long ldb,
                  int bc0, int N, int M, float* clo, float* chi) {
      TGemmArgs t{};
      t.S = E;
      t.seg_start = B->offsets;
      t.seg_count = B->counts;
      t.a = A;
      t.a_dtype = adt;
      t.lda = lda;
      t.a_c0 = ac0;
      t.a_map = amap;
      t.a_div = adiv;
      t.b = Bm;
      t.ldb = ldb;
      t.b_c0 = bc0;
      t.N = N;
      t.M = M;
      t.c_lo = clo;
      t.c_hi = chi;
      t.c_sstride = (long)M * r;
      t.ldc = r;
      t.n_store = r;
      ok(launch_tgemm(ty, t, st));
    };
    // dA1_p = X^T q_p (both input projections in one pass over X)
    tg(X, c.x_dtype, d, 0, B->arow, k, B->q, 64, 0, Pin * 16, d, gr->dA[0], Pin > 1 ? gr->dA[1] : nullptr);
    // dB1_p = dz_p^T u_p
    for (int p = 0; p < Pin; ++p)
      tg(B->dz, ty, (long)Pin * f, p * f, nullptr, 1, B->ua, 64, p * 16, 16, f, gr->dB[p], nullptr);
    // dA2 = (w h)^T e, dB2 = dY^T (w h A2)
    tg(B->wh, ty, f, 0, nullptr, 1, B->ea, 16, 0, 16, f, gr->dA[P - 1], nullptr);
    tg(dY, c.x_dtype, d, 0, B->arow, k, B->wu2, 16, 0, 16, d, gr->dB[P - 1], nullptr);
  }
  if (e != hipSuccess) return hip_fail(h, e, "backward launch");
  return MOE_OK;
}

}  // extern "C"

