// Internal interface of the C ABI implementation, shared by api.hip
// (create, route, forward), backward.hip (moe_backward) and offload.hip
// (idle-group offload): the handle, its forward workspace, and the helpers
// and pieces of the forward pass the other two reuse.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "moe.h"
#include "pack.h"
#include "train.h"

namespace cefn_api {
constexpr int kStages = 7;     // profiled stages of a forward pass
constexpr int kMaxSplits = 4;  // k splits of the down projection (ypart holds this many)
}  // namespace cefn_api

// Workspace of one forward pass, carved out of one device buffer for a
// capacity of T_cap tokens: the handle's own buffer (carved once for T_max)
// or the static scratch array of the no-allocation entry point (carved per
// call for that call's T).  Only the per-chunk counters cc must be zero when
// a pass starts; every other piece is written before it is read.
struct Workspace {
  long T_cap = 0;
  int *idx = nullptr, *gidx = nullptr, *counts = nullptr, *offsets = nullptr;
  int *gcounts = nullptr, *goffsets = nullptr, *garow = nullptr, *garow_sorted = nullptr;
  int* cc = nullptr;  // per-chunk counters: [nch_e_max][E] then [nch_g_max][G]
  int nch_e_max = 0, nch_g_max = 0, cc_n = 0;
  uint16_t* X16 = nullptr;  // fp16 copy of bf16 activations (fp16 MFMAs)
  float* w = nullptr;
  float* L = nullptr;   // router scores (k-split partials)
  void* U = nullptr;    // [T*kg][NU]
  float* V = nullptr;   // [T*kg][NV]
  float* Vp = nullptr;  // [G1 column tiles][T_cap*kg][ke][16]
  int nt1k = 0;         // column tiles of the k-split G1 (0: its partials do not fit)
  void* H = nullptr;    // [T*kg][f]
  float* ypart = nullptr;
};

struct moe_handle {
  moe_config cfg{};
  int E = 0, k = 0, P = 0, P_in = 0, mma = 0, NU = 0, NV = 0;
  int device = 0;
  bool dirty = false;
  // weights
  float *Wr = nullptr, *gbias = nullptr, *ebias = nullptr;
  uint16_t* Wb = nullptr;  // bf16 parts of Wr (16-bit activations)
  int NCp = 0;         // router score columns, padded to 32
  float* L = nullptr;  // router scores (k-split partials)
  void *W1 = nullptr, *W2 = nullptr, *At = nullptr, *B1 = nullptr, *Ad = nullptr, *Bd = nullptr;
  uint16_t *At_s = nullptr, *B1_s = nullptr, *Ad_s = nullptr, *Bd_s = nullptr;
  long w1_gs = 0, w2_gs = 0, at_gs = 0, at_sgs = 0, bd_gs = 0;
  Workspace ws;         // the handle's own workspace, carved for T_max
  int nt1 = 0;          // column tiles of gemm1 (partials of V per row)
  std::vector<void*> allocs;
  int64_t weight_bytes = 0;
  // tile rows and stage depth per GEMM (0 = chosen per call); set from the
  // tile overrides read from CEFN_BM_{U,G1,G2} (token rows per tile) and
  // CEFN_KS_G2 (k splits of the down projection) at create, for tuning
  int bm_env[3] = {0, 0, 0}, ks_env = 0;
  int g2k_env = -1;  // CEFN_G2K: 1 / 0 forces the in-workgroup k split of G2 on / off
  int g1k_env = -1;  // CEFN_G1K: 1 / 2 forces the k-split tiles of G1 (d in four / in two), 0 off
  int ut_env = -1;   // CEFN_UT: 1 / 0 forces the tile-engine U GEMM on / off
  int gsort_env = -1;  // CEFN_GSORT: 1 / 0 forces the per-group row sort on / off
  int tail_env = -1;   // CEFN_TAIL_SLOTS: 0 turns G2's last-round split off, N > 0 sets its round size
  // profiling
  bool prof = false;
  int prof_max = 0, prof_calls = 0, prof_mask = -1;
  std::vector<hipEvent_t> ev;          // [prof_max][kStages][2]
  std::vector<unsigned char> ev_used;  // [prof_max][kStages]
  struct BwdState* bwd = nullptr;      // backward-pass layouts and workspace (built on first use)
  struct OffloadState* off = nullptr;  // idle-group offload (moe_offload_enable)
};

namespace cefn_api {

#define TRY(x)            \
  do {                    \
    int rc_ = (x);        \
    if (rc_) return rc_;  \
  } while (0)

int fail(int code, const char* fmt, ...);
int hip_fail(moe_handle* h, hipError_t e, const char* what);
int elem_bytes(int dt);
void dims(const moe_config& c, int p, int& din, int& dout);
int max_mtiles(int T, int kg, int G, int bm);

template <class T>
int dalloc(moe_handle* h, T** p, size_t n) {
  *p = nullptr;
  if (n == 0) return MOE_OK;
  void* q = nullptr;
  if (hipMalloc(&q, n * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_OOM, "hipMalloc of %zu bytes failed", n * sizeof(T));
  }
  h->allocs.push_back(q);
  *p = static_cast<T*>(q);
  return MOE_OK;
}

struct Prof {
  moe_handle* h;
  hipStream_t st;
  int call;
  bool on(int s) const { return call >= 0 && ((h->prof_mask >> s) & 1); }
  void begin(int s) {
    if (on(s)) (void)hipEventRecord(h->ev[((size_t)call * kStages + s) * 2], st);
  }
  void end(int s) {
    if (on(s)) {
      (void)hipEventRecord(h->ev[((size_t)call * kStages + s) * 2 + 1], st);
      h->ev_used[(size_t)call * kStages + s] = 1;
    }
  }
};

// Where the routing pass left the lists the GEMMs read.
struct RouteLive {
  int *gcounts, *goffsets, *idx, *gidx;
  float* w;
};

int run_route(moe_handle* h, Workspace& ws, const void* X, int T, const moe_route_out* ro, bool need_experts,
              hipStream_t st, Prof& pf, RouteLive& live);

// Where one residual factor (projection p, A or B, expert i) lives in the
// device layouts, in the terms of the decode kernel (kinds: 0 At, 1 B1,
// 2 Ad, 3 Bd).
struct FactorLoc {
  int kind, n, aux0, aux1;
  const void* src;
  const uint16_t* sc;
  long base, sbase;
};

FactorLoc locate_factor(const moe_handle* h, int proj, int which, int expert);

// State a forward pass carries from its routing to its GEMMs and combine.
struct FwdState {
  Prof pf;
  RouteLive live;
  const int* garow;
  bool gsorted;
  const void* xg;  // activations the row GEMMs read (X, or its fp16 copy)
  int xt;
  int splits;
};

int fwd_prelude(moe_handle* h, Workspace& ws, const void* X, int T, const moe_route_out* routing, hipStream_t st,
                FwdState& fs);
int fwd_gemms(moe_handle* h, Workspace& ws, const void* X, int T, void* Y, hipStream_t st, FwdState& fs,
              const int* gcounts, const int* gslot);
int fwd_combine(moe_handle* h, Workspace& ws, int T, void* Y, hipStream_t st, FwdState& fs);

// Release the backward / offload state of a handle (backward.hip, offload.hip).
void delete_bwd(moe_handle* h);
void delete_offload(moe_handle* h);

}  // namespace cefn_api
