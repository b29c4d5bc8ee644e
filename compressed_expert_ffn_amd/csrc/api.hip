// C ABI of the compressed-expert MoE FFN layer (declared in include/moe.h).
//
// moe_create validates the shape, quantises and re-lays-out the weights
// (pack.cpp) and allocates a workspace sized for T_max tokens.  moe_forward
// enqueues, on the caller's stream and without host synchronisation:
//   router    two-level top-k and gate weights, assignment counts per chunk
//   scatter   counts -> offsets -> stable per-expert and per-group lists
//   ugemm     u = x A for every expert of each chosen group   (r > 0)
//   gemm1     base input projections once per (token, group) + residual,
//             activation, gate-weighted sum and h A_down in the epilogue
//   gemm2     base output projection + stacked residual tail
//   combine   sum over chosen groups                           (kg > 1)
// The per-chunk counters are zero between calls: create clears them and the
// last GEMM of every forward (or a small clear kernel after moe_route)
// clears them again.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "api_internal.h"

using namespace cefn;
using namespace cefn_api;

namespace cefn_api {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

long roundup(long x, long m) { return (x + m - 1) / m * m; }

const char* kStageNames[] = {"router", "scatter", "ugemm", "gemm1", "vreduce", "gemm2", "combine"};

}  // namespace cefn_api

namespace cefn {
int report_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
}  // namespace cefn

// Workspace of the no-allocation forward pass (moe_forward_noalloc): one
// array in every device's memory, held until the process ends.  Host code
// never uses the name itself: on each device the array's address comes from
// hipGetSymbolAddress (with that device current) and is kept per device.
constexpr size_t kScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace cefn_api {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Address of this device's scratch array (looked up once per device, with
// that device current).
int scratch_for_device(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace cefn_api

namespace cefn_api {

int elem_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

int validate(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "null config");
  if (c->T_max < 0 || c->d <= 0 || c->f <= 0 || c->G <= 0 || c->K <= 0 || c->top_groups <= 0 ||
      c->top_experts <= 0 || c->r < 0)
    return fail(MOE_ERR_INVALID_ARG, "config sizes must be positive (r >= 0, T_max >= 0)");
  if (c->act != MOE_ACT_GELU_TANH && c->act != MOE_ACT_SWIGLU)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation %d", c->act);
  if (c->x_dtype < 0 || c->x_dtype > 2 || c->base_dtype < 0 || c->base_dtype > 2)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (c->resid < 0 || c->resid > 3) return fail(MOE_ERR_INVALID_ARG, "unknown residual kind");
  if (c->top_groups > c->G) return fail(MOE_ERR_INVALID_ARG, "top_groups %d > G %d", c->top_groups, c->G);
  if (c->top_experts > c->K) return fail(MOE_ERR_INVALID_ARG, "top_experts %d > K %d", c->top_experts, c->K);
  if ((c->r == 0) != (c->resid == MOE_RESID_NONE))
    return fail(MOE_ERR_INVALID_ARG, "r == 0 exactly when the residual kind is NONE");
  const long E = (long)c->G * c->K;
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "G*K = %ld > 1024", E);
  if (c->G > 256 || c->K > 256) return fail(MOE_ERR_UNSUPPORTED, "G and K must be <= 256");
  if (c->top_groups > MAX_KG) return fail(MOE_ERR_UNSUPPORTED, "top_groups > %d", MAX_KG);
  if (c->top_groups * c->top_experts > MAX_SLOTS)
    return fail(MOE_ERR_UNSUPPORTED, "top_groups*top_experts > %d", MAX_SLOTS);
  if (c->r > RPAD) return fail(MOE_ERR_UNSUPPORTED, "r > %d", RPAD);
  if (c->r > 0 && c->K > 64) return fail(MOE_ERR_UNSUPPORTED, "residual experts need K <= 64");
  if (c->d % 64 || c->f % 64) return fail(MOE_ERR_UNSUPPORTED, "d and f must be multiples of 64");
  const int x = c->x_dtype, b = c->base_dtype;
  const bool pair_ok = (x == MOE_F32 && b == MOE_F32) || (x == MOE_F16 && b == MOE_F16) ||
                       (x == MOE_BF16 && b == MOE_BF16) || (x == MOE_BF16 && b == MOE_F16);
  if (!pair_ok) return fail(MOE_ERR_UNSUPPORTED, "unsupported (x, base) dtype pair (%d, %d)", x, b);
  if (c->resid == MOE_RESID_F32 && b != MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "F32 residual needs an F32 base");
  if (c->resid == MOE_RESID_F16 && b != MOE_F16) return fail(MOE_ERR_UNSUPPORTED, "F16 residual needs an F16 base");
  if (c->resid == MOE_RESID_INT4_G32 && b == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "INT4 residual needs an F16 or BF16 base");
  return MOE_OK;
}

void dims(const moe_config& c, int p, int& din, int& dout) {
  const int P = c.act == MOE_ACT_SWIGLU ? 3 : 2;
  if (p < P - 1) {
    din = c.d;
    dout = c.f;
  } else {
    din = c.f;
    dout = c.d;
  }
}

void compute_stats(const moe_config& c, moe_stats_t* s) {
  const int P = c.act == MOE_ACT_SWIGLU ? 3 : 2;
  const long E = (long)c.G * c.K;
  int64_t params = 0, dense = 0, bytes = 0;
  for (int p = 0; p < P; ++p) {
    int di, dn;
    dims(c, p, di, dn);
    params += (int64_t)c.G * di * dn + E * c.r * (int64_t)(di + dn);
    dense += E * (int64_t)di * dn;
    bytes += (int64_t)c.G * di * dn * elem_bytes(c.base_dtype);
    if (c.resid == MOE_RESID_INT4_G32)
      bytes += E * ((int64_t)(di + dn) * c.r / 2 + (int64_t)(di + dn) / 32 * c.r * 2);
    else if (c.resid != MOE_RESID_NONE)
      bytes += E * (int64_t)(di + dn) * c.r * (c.resid == MOE_RESID_F32 ? 4 : 2);
  }
  s->stored_params = params;
  s->dense_equiv_params = dense;
  s->stored_bytes = bytes;
}


// Lay the workspace for T tokens out from `base` (256-byte aligned pieces);
// returns the bytes it spans.  base == nullptr only measures.
size_t carve_workspace(const moe_handle* h, long T, char* base, Workspace* ws) {
  const moe_config& c = h->cfg;
  const long k = h->k, kg = c.top_groups;
  const size_t es = elem_bytes(h->mma);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  *ws = Workspace{};
  ws->T_cap = T;
  ws->nch_e_max = (int)((T * k + CHUNK - 1) / CHUNK);
  ws->nch_g_max = (int)((T * kg + CHUNK - 1) / CHUNK);
  ws->cc_n = ws->nch_e_max * h->E + ws->nch_g_max * c.G;
  ws->idx = reinterpret_cast<int*>(take(sizeof(int) * (T * k + 1)));
  ws->w = reinterpret_cast<float*>(take(sizeof(float) * (T * k + 1)));
  ws->gidx = reinterpret_cast<int*>(take(sizeof(int) * (T * kg + 1)));
  ws->counts = reinterpret_cast<int*>(take(sizeof(int) * h->E));
  ws->offsets = reinterpret_cast<int*>(take(sizeof(int) * (h->E + 1)));
  ws->gcounts = reinterpret_cast<int*>(take(sizeof(int) * c.G));
  ws->goffsets = reinterpret_cast<int*>(take(sizeof(int) * (c.G + 1)));
  ws->garow = reinterpret_cast<int*>(take(sizeof(int) * (T * kg + 1)));
  if (c.x_dtype == MOE_BF16 && h->mma == MOE_F16) ws->X16 = reinterpret_cast<uint16_t*>(take(2 * (T * c.d + 8)));
  if (c.r > 0 && c.K > 1 && c.top_experts < c.K) ws->garow_sorted = reinterpret_cast<int*>(take(sizeof(int) * (T * kg + 1)));
  ws->cc = reinterpret_cast<int*>(take(sizeof(int) * ((size_t)ws->cc_n + 1)));
  {
    // score buffer: the largest nsplit * T over the batch sizes up to T
    long lmax = 0;
    for (long t = 32; t < T + 32; t += 32) {
      const long tt = std::min<long>(t, std::max<long>(T, 1));
      lmax = std::max(lmax, router_splits((int)tt, c.d, h->NCp) * tt);
    }
    ws->L = reinterpret_cast<float*>(take(sizeof(float) * ((size_t)lmax * h->NCp + 4)));
  }
  if (c.r > 0) {
    ws->U = take(T * kg * h->NU * es + 16);
    ws->V = reinterpret_cast<float*>(take(sizeof(float) * (T * kg * h->NV + 4)));
    // the k-split G1 writes one V partial per 64 columns: room for those
    // when it stays under 256 MiB (the layouts that use it have few rows)
    const int nt1k = h->P_in * c.f / 64;
    const size_t per_tile = (size_t)T * kg * c.top_experts * RPAD;
    ws->nt1k = per_tile * nt1k * sizeof(float) <= ((size_t)256 << 20) ? nt1k : 0;
    ws->Vp = reinterpret_cast<float*>(take(sizeof(float) * ((size_t)std::max(h->nt1, ws->nt1k) * per_tile + 4)));
  }
  ws->H = take(T * kg * (long)c.f * es + 16);
  ws->ypart = reinterpret_cast<float*>(take(sizeof(float) * ((size_t)kMaxSplits * T * kg * c.d + 4)));
  return off;
}

template <class T>
int upload(moe_handle* h, T** dst, const std::vector<T>& src) {
  int rc = dalloc(h, dst, src.size());
  if (rc) return rc;
  if (src.empty()) return MOE_OK;
  if (hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return fail(MOE_ERR_HIP, "hipMemcpy to device failed");
  h->weight_bytes += src.size() * sizeof(T);
  return MOE_OK;
}

template <class T>
int upload_raw(moe_handle* h, void** dst, const std::vector<T>& src) {
  T* p = nullptr;
  int rc = upload(h, &p, src);
  *dst = p;
  return rc;
}

// Build every device weight array.  TS is the storage type of the MFMA
// dtype: float (F32) or uint16_t bits (F16/BF16), which is also the storage
// type of the base and of F32/F16 residuals.
template <class TS>
int build_weights(moe_handle* h, const moe_weights* w) {
  const moe_config& c = h->cfg;
  const int G = c.G, K = c.K, E = h->E, P = h->P, Pin = h->P_in, d = c.d, f = c.f, r = c.r;
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  auto base_ptr = [&](int p) { return static_cast<const TS*>(w->base[p]); };

  // base input projections, gate/up interleaved in 32-column blocks for SwiGLU
  {
    const int N = Pin * f;
    std::vector<TS> buf((size_t)G * N * d);
    h->w1_gs = (long)N * d;
    for (int g = 0; g < G; ++g) {
      pack_frag(buf.data() + (size_t)g * N * d, N, d, true, [&](int n, int k) -> TS {
        int p = 0, col = n;
        if (swiglu) {
          const int blk = n / 32;
          p = blk & 1;
          col = (blk >> 1) * 32 + (n & 31);
        }
        return base_ptr(p)[((size_t)g * d + k) * f + col];
      });
    }
    TRY(upload_raw(h, &h->W1, buf));
  }
  // base output projection [f][d]
  {
    std::vector<TS> buf((size_t)G * d * f);
    h->w2_gs = (long)d * f;
    for (int g = 0; g < G; ++g)
      pack_frag(buf.data() + (size_t)g * d * f, d, f, true,
                [&](int n, int k) -> TS { return base_ptr(P - 1)[((size_t)g * f + k) * d + n]; });
    TRY(upload_raw(h, &h->W2, buf));
  }
  if (r == 0) return MOE_OK;

  const int NU = h->NU, NV = h->NV;
  if (c.resid == MOE_RESID_INT4_G32) {
    // quantise every factor once
    std::vector<Q4> qa((size_t)P * E), qb((size_t)P * E);
    for (int p = 0; p < P; ++p) {
      int di, dn;
      dims(c, p, di, dn);
      const float* Ap = static_cast<const float*>(w->A[p]);
      const float* Bp = static_cast<const float*>(w->B[p]);
      parallel_for(E, [&](int i) {
        qa[(size_t)p * E + i] = quantize_g32(Ap + (size_t)i * di * r, di, r);
        qb[(size_t)p * E + i] = quantize_g32(Bp + (size_t)i * dn * r, dn, r);
      });
    }
    auto QA = [&](int p, int i) -> const Q4& { return qa[(size_t)p * E + i]; };
    auto QB = [&](int p, int i) -> const Q4& { return qb[(size_t)p * E + i]; };
    // At: [G] frag(NU, d) + scales [G][NU/32][d/32][32]
    {
      std::vector<uint32_t> wbuf((size_t)G * NU * d / 8);
      std::vector<uint16_t> sbuf((size_t)G * (NU / 32) * (d / 32) * 32, 0);
      h->at_gs = (long)NU * d / 8;
      h->at_sgs = (long)(NU / 32) * (d / 32) * 32;
      for (int g = 0; g < G; ++g) {
        auto col = [&](int n, int& j, int& p, int& rho) {
          j = n / (Pin * RPAD);
          p = (n / RPAD) % Pin;
          rho = n % RPAD;
          return j < K && rho < r;
        };
        pack_frag_int4(wbuf.data() + (size_t)g * h->at_gs, NU, d, true, [&](int n, int k) {
          int j, p, rho;
          return col(n, j, p, rho) ? QA(p, g * K + j).code(k, rho) : 0;
        });
        for (int n = 0; n < NU; ++n) {
          int j, p, rho;
          if (!col(n, j, p, rho)) continue;
          for (int kb = 0; kb < d / 32; ++kb)
            sbuf[(size_t)g * h->at_sgs + ((size_t)(n / 32) * (d / 32) + kb) * 32 + (n % 32)] =
                QA(p, g * K + j).scale(kb * 32, rho);
        }
      }
      TRY(upload_raw(h, &h->At, wbuf));
      TRY(upload(h, &h->At_s, sbuf));
    }
    // B1: [E][Pin] frag(f, 16) + scales [E][Pin][f/32][16]
    {
      std::vector<uint32_t> wbuf((size_t)E * Pin * f * 16 / 8);
      std::vector<uint16_t> sbuf((size_t)E * Pin * (f / 32) * RPAD, 0);
      for (int i = 0; i < E; ++i)
        for (int p = 0; p < Pin; ++p) {
          const Q4& q = QB(p, i);
          pack_frag_int4(wbuf.data() + (size_t)(i * Pin + p) * f * 2, f, RPAD, false,
                         [&](int n, int k) { return k < r ? q.code(n, k) : 0; });
          for (int fb = 0; fb < f / 32; ++fb)
            for (int rho = 0; rho < r; ++rho)
              sbuf[((size_t)(i * Pin + p) * (f / 32) + fb) * RPAD + rho] = q.scale(fb * 32, rho);
        }
      TRY(upload_raw(h, &h->B1, wbuf));
      TRY(upload(h, &h->B1_s, sbuf));
    }
    // Ad: [E][f/32][2][64] words (see ad_row) + scales [E][f/32][16]
    {
      std::vector<uint32_t> wbuf((size_t)E * (f / 32) * 2 * 64);
      std::vector<uint16_t> sbuf((size_t)E * (f / 32) * RPAD, 0);
      for (int i = 0; i < E; ++i) {
        const Q4& q = QA(P - 1, i);
        for (int fb = 0; fb < f / 32; ++fb) {
          for (int st = 0; st < 2; ++st)
            for (int lane = 0; lane < 64; ++lane) {
              const int rho = lane & 31;
              uint32_t word = 0;
              for (int e = 0; e < 8; ++e) {
                const int kk = fb * 32 + ad_row(st, lane >> 5, e);
                const int qv = rho < r ? q.code(kk, rho) : 0;
                word |= static_cast<uint32_t>(qv + 8) << (4 * e);
              }
              wbuf[(((size_t)i * (f / 32) + fb) * 2 + st) * 64 + lane] = word;
            }
          for (int rho = 0; rho < r; ++rho) sbuf[((size_t)i * (f / 32) + fb) * RPAD + rho] = q.scale(fb * 32, rho);
        }
      }
      TRY(upload_raw(h, &h->Ad, wbuf));
      TRY(upload(h, &h->Ad_s, sbuf));
    }
    // Bd: [G] frag(d, NV) + scales [E][d/32][16]
    {
      std::vector<uint32_t> wbuf((size_t)G * d * NV / 8);
      std::vector<uint16_t> sbuf((size_t)E * (d / 32) * RPAD, 0);
      h->bd_gs = (long)d * NV / 8;
      for (int g = 0; g < G; ++g)
        pack_frag_int4(wbuf.data() + (size_t)g * h->bd_gs, d, NV, true, [&](int n, int k) {
          const int j = k / RPAD, rho = k % RPAD;
          return (j < K && rho < r) ? QB(P - 1, g * K + j).code(n, rho) : 0;
        });
      for (int i = 0; i < E; ++i)
        for (int nb = 0; nb < d / 32; ++nb)
          for (int rho = 0; rho < r; ++rho)
            sbuf[((size_t)i * (d / 32) + nb) * RPAD + rho] = QB(P - 1, i).scale(nb * 32, rho);
      TRY(upload_raw(h, &h->Bd, wbuf));
      TRY(upload(h, &h->Bd_s, sbuf));
    }
    return MOE_OK;
  }

  // F32 / F16 residuals stored in the MFMA type directly
  auto Aval = [&](int p, int i, int k, int rho) -> TS {
    int di, dn;
    dims(c, p, di, dn);
    return static_cast<const TS*>(w->A[p])[((size_t)i * di + k) * r + rho];
  };
  auto Bval = [&](int p, int i, int n, int rho) -> TS {
    int di, dn;
    dims(c, p, di, dn);
    return static_cast<const TS*>(w->B[p])[((size_t)i * dn + n) * r + rho];
  };
  const TS zero = TS(0);
  {
    std::vector<TS> buf((size_t)G * NU * d);
    h->at_gs = (long)NU * d;
    for (int g = 0; g < G; ++g)
      pack_frag(buf.data() + (size_t)g * NU * d, NU, d, true, [&](int n, int k) -> TS {
        const int j = n / (Pin * RPAD), p = (n / RPAD) % Pin, rho = n % RPAD;
        return (j < K && rho < r) ? Aval(p, g * K + j, k, rho) : zero;
      });
    TRY(upload_raw(h, &h->At, buf));
  }
  {
    std::vector<TS> buf((size_t)E * Pin * f * RPAD);
    for (int i = 0; i < E; ++i)
      for (int p = 0; p < Pin; ++p)
        pack_frag(buf.data() + (size_t)(i * Pin + p) * f * RPAD, f, RPAD, false,
                  [&](int n, int k) -> TS { return k < r ? Bval(p, i, n, k) : zero; });
    TRY(upload_raw(h, &h->B1, buf));
  }
  {
    std::vector<TS> buf((size_t)E * (f / 32) * 2 * 64 * 8);
    for (int i = 0; i < E; ++i)
      for (int fb = 0; fb < f / 32; ++fb)
        for (int st = 0; st < 2; ++st)
          for (int lane = 0; lane < 64; ++lane)
            for (int e = 0; e < 8; ++e) {
              const int rho = lane & 31, kk = fb * 32 + ad_row(st, lane >> 5, e);
              buf[((((size_t)i * (f / 32) + fb) * 2 + st) * 64 + lane) * 8 + e] = rho < r ? Aval(P - 1, i, kk, rho) : zero;
            }
    TRY(upload_raw(h, &h->Ad, buf));
  }
  {
    std::vector<TS> buf((size_t)G * d * NV);
    h->bd_gs = (long)d * NV;
    for (int g = 0; g < G; ++g)
      pack_frag(buf.data() + (size_t)g * d * NV, d, NV, true, [&](int n, int k) -> TS {
        const int j = k / RPAD, rho = k % RPAD;
        return (j < K && rho < r) ? Bval(P - 1, g * K + j, n, rho) : zero;
      });
    TRY(upload_raw(h, &h->Bd, buf));
  }
  return MOE_OK;
}

// Token rows per tile for a grouped GEMM with `rows` rows and `ntiles`
// column tiles of 256.  Bigger tiles reuse each weight fragment over more
// tokens (fewer bytes per MFMA) but give fewer workgroups; the estimate
// below charges each choice its number of rounds over the 256 compute units
// times the tile height, discounted by the main loop's measured efficiency
// at that height.
int pick_bm(const moe_handle* h, int which, int rows, int ntiles, int splits) {
  const bool f32 = h->mma == MOE_F32;
  if (h->bm_env[which]) return h->bm_env[which];
  static const int cand[4] = {256, 128, 64, 32};
  // relative MFMA efficiency of the tile heights (main loop measured at
  // 50% of peak with 256 rows, 46% with 128; the product's layers agree)
  static const float eff[4] = {1.0f, 0.88f, 0.75f, 0.5f};
  int best = 32;
  float best_cost = 1e30f;
  for (int i = 0; i < 4; ++i) {
    const int bm = cand[i];
    if (f32 && bm > 64) continue;
    // GELU keeps two f-blocks of h per wavefront: up to 128 rows without spills
    if (which == GK_G1 && h->cfg.act != MOE_ACT_SWIGLU && bm > 128) continue;
    if (gemm_lds(which, h->mma, bm, h->cfg.K, h->cfg.top_experts) > 160 * 1024) continue;
    // row tiles: every group's last tile is partial (counted as half)
    const long mt = (rows + bm - 1) / bm + h->cfg.G / 2;
    const long tiles = mt * ntiles * splits;
    int occ = bm <= 64 ? 2 : 1;  // workgroups per compute unit
    float e = eff[i];
    if (which == GK_G1 && bm == 128 && !f32 && h->cfg.act == MOE_ACT_SWIGLU) {
      // the SwiGLU gemm1 at 128 rows fits two workgroups per compute unit,
      // so one's epilogue overlaps the other's main loop: measured 6-18%
      // faster than 256-row tiles on the fp16, flat bf16 and INT4 layers
      occ = 2;
      e = 1.1f;
    }
    const long rounds = (tiles + 256L * occ - 1) / (256L * occ);
    const float cost = rounds * (float)bm * occ / e / splits;
    if (cost < best_cost) {
      best_cost = cost;
      best = bm;
    }
  }
  return best;
}

// k splits of the down projection and its tile height together, from a
// small time model: each round of workgroups costs one tile's MFMA work at
// a third of the chip's per-unit peak (times the tile height's efficiency),
// and any split (or more than one chosen group) adds the partial sums that
// the combine kernel reads back, at 5 TB/s.  Each split keeps at least 8
// stages of 64.
void pick_g2(const moe_handle* h, int rows, int ntiles, int& bm, int& splits) {
  const moe_config& c = h->cfg;
  const int kt = c.f / 64;
  const double unit_rate = 2.5e15 / 256 * 0.35;  // flop/s of one compute unit
  double best = 1e30;
  bm = 128;
  splits = 1;
  if ((long)rows < 32L * c.G && !h->ks_env && !h->bm_env[GK_G2]) {
    // under 32 rows per group (decode-shaped): every tile streams its
    // weights from HBM whatever the split, so splits only add partial sums;
    // 32-row tiles, one split (measured on the decode layer: 41 us against
    // 51 us for the split the model below picks)
    bm = 32;
    return;
  }
  for (int s = 1; s <= kMaxSplits; ++s) {
    if (h->ks_env && s != h->ks_env) continue;
    if (s > 1 && kt / s < 8) break;
    for (int b : {256, 128, 64, 32}) {
      if (h->bm_env[GK_G2] && b != h->bm_env[GK_G2]) continue;
      if (h->mma == MOE_F32 && b > 64) continue;
      const long mt = (rows + b - 1) / b + c.G / 2;
      // 128-row tiles of 16-bit types run two workgroups per compute unit
      // (measured 5-15% faster than 256-row tiles on the large layers)
      const bool two = b <= 64 || (b == 128 && h->mma != MOE_F32);
      const long tiles = mt * ntiles * s;
      const double eff = b >= 256 ? 1.0 : b == 128 ? (two ? 1.05 : 0.88) : b == 64 ? 0.75 : 0.5;
      const double wg = 2.0 * b * 256 * ((double)c.f / s) / (unit_rate * eff);  // one workgroup alone
      // the busiest compute unit's share of workgroups: two resident ones
      // share its MFMA pipe, so residency hides latency (in eff) but does
      // not add throughput
      double t = (double)((tiles + 255) / 256) * wg;
      // one split: a last round at most half full is cut along k over the
      // whole chip (see the launch), so the rounds count as a fraction,
      // plus a tenth of a round for the pieces
      const long slots = b == 128 ? 512 : 256;
      const bool tail = s == 1 && h->mma != MOE_F32 && b >= 128 && h->tail_env != 0 && tiles > slots &&
                        2 * (tiles % slots) <= slots;
      if (tail) t = ((double)tiles / 256 + 0.1) * wg;
      if (s > 1 || c.top_groups > 1) t += ((double)s * rows * c.d * 4 + (double)rows / c.top_groups * c.d * 2) / 5e12;
      if (t < best) {
        best = t;
        bm = b;
        splits = s;
      }
    }
  }
}

int max_mtiles(int T, int kg, int G, int bm) {
  const long rows = (long)T * kg;
  return (int)((rows + bm - 1) / bm + std::min<long>(G, rows));
}

int hip_fail(moe_handle* h, hipError_t e, const char* what) {
  h->dirty = true;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Weights handed over as device pointers: read every array back into host
// buffers (owned by `store`) and point a host-side copy of the struct at them,
// so the packing below has one source form.
int weights_to_host(const moe_config& c, const moe_weights* w, moe_weights* hw,
                    std::vector<std::vector<char>>& store) {
  *hw = *w;
  hw->on_device = 0;
  const int P = c.act == MOE_ACT_SWIGLU ? 3 : 2;
  const long E = (long)c.G * c.K;
  auto pull = [&](const void* src, size_t bytes, const void** dst) -> int {
    if (!src) {
      *dst = nullptr;
      return MOE_OK;
    }
    store.emplace_back(bytes);
    if (hipMemcpy(store.back().data(), src, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MOE_ERR_INVALID_ARG, "on_device weights: copy from device failed (not a device pointer?)");
    }
    *dst = store.back().data();
    return MOE_OK;
  };
  const void* t = nullptr;
  TRY(pull(w->W_grp, sizeof(float) * c.d * c.G, &t));
  hw->W_grp = static_cast<const float*>(t);
  TRY(pull(c.K > 1 ? w->W_exp : nullptr, sizeof(float) * c.G * (size_t)c.d * c.K, &t));
  hw->W_exp = static_cast<const float*>(t);
  TRY(pull(w->group_bias, sizeof(float) * c.G, &t));
  hw->group_bias = static_cast<const float*>(t);
  TRY(pull(c.K > 1 ? w->expert_bias : nullptr, sizeof(float) * E, &t));
  hw->expert_bias = static_cast<const float*>(t);
  const size_t rb = c.resid == MOE_RESID_F16 ? 2 : 4;
  for (int p = 0; p < P; ++p) {
    int di, dn;
    dims(c, p, di, dn);
    TRY(pull(w->base[p], (size_t)c.G * di * dn * elem_bytes(c.base_dtype), &hw->base[p]));
    if (c.r > 0) {
      TRY(pull(w->A[p], (size_t)E * di * c.r * rb, &hw->A[p]));
      TRY(pull(w->B[p], (size_t)E * dn * c.r * rb, &hw->B[p]));
    } else {
      hw->A[p] = hw->B[p] = nullptr;
    }
  }
  return MOE_OK;
}

}  // namespace cefn_api

namespace cefn_api {

// router + scatter into the workspace (and the caller's buffers where given)
int run_route(moe_handle* h, Workspace& ws, const void* X, int T, const moe_route_out* ro, bool need_experts,
              hipStream_t st, Prof& pf, RouteLive& live) {
  const moe_config& c = h->cfg;
  hipError_t e;
  if (h->dirty && &ws == &h->ws) {
    e = launch_zero(ws.cc, ws.cc_n, st);
    if (e != hipSuccess) return hip_fail(h, e, "clear counters");
    h->dirty = false;
  }
  int* idx = (ro && ro->idx) ? ro->idx : ws.idx;
  float* wts = (ro && ro->w) ? ro->w : ws.w;
  int* gidx = (ro && ro->gidx) ? ro->gidx : ws.gidx;
  RouteArgs ra{};
  ra.X = X;
  ra.T = T;
  ra.d = c.d;
  ra.G = c.G;
  ra.K = c.K;
  ra.kg = c.top_groups;
  ra.ke = c.top_experts;
  ra.k = h->k;
  ra.E = h->E;
  ra.Wr = h->Wr;
  ra.Wb = h->Wb;
  ra.NCp = h->NCp;
  ra.L = ws.L;
  ra.nsplit = router_splits(T, c.d, h->NCp);
  ra.gbias = h->gbias;
  ra.ebias = h->ebias;
  ra.idx = idx;
  ra.w = wts;
  ra.gidx = gidx;
  ra.ccount = ws.cc;
  ra.cgcount = ws.cc + (size_t)ws.nch_e_max * h->E;
  // the forward pass needs only the group lists; expert-level counts,
  // offsets and perm are built when the caller asks for routing outputs
  ra.count_experts = need_experts ? 1 : 0;
  pf.begin(0);
  e = launch_router(c.x_dtype, ra, st);
  if (e != hipSuccess) return hip_fail(h, e, "router launch");
  pf.end(0);
  ScatterArgs sa{};
  sa.T = T;
  sa.k = h->k;
  sa.kg = c.top_groups;
  sa.E = h->E;
  sa.G = c.G;
  sa.idx = idx;
  sa.gidx = gidx;
  sa.ccount = ra.ccount;
  sa.cgcount = ra.cgcount;
  sa.nch_e = (int)(((long)T * h->k + CHUNK - 1) / CHUNK);
  sa.nch_g = (int)(((long)T * c.top_groups + CHUNK - 1) / CHUNK);
  sa.counts = (ro && ro->counts) ? ro->counts : ws.counts;
  sa.offsets = (ro && ro->offsets) ? ro->offsets : ws.offsets;
  sa.perm = (ro && ro->perm) ? ro->perm : nullptr;
  sa.gcounts = (ro && ro->gcounts) ? ro->gcounts : ws.gcounts;
  sa.goffsets = (ro && ro->goffsets) ? ro->goffsets : ws.goffsets;
  sa.gperm = (ro && ro->gperm) ? ro->gperm : nullptr;
  sa.garow = ws.garow;
  sa.do_experts = ra.count_experts;
  pf.begin(1);
  e = launch_scatter(sa, st);
  if (e != hipSuccess) return hip_fail(h, e, "scatter launch");
  pf.end(1);
  // the GEMMs read the group lists from wherever the scatter put them
  live.gcounts = sa.gcounts;
  live.goffsets = sa.goffsets;
  live.idx = idx;
  live.w = wts;
  live.gidx = gidx;
  return MOE_OK;
}

}  // namespace cefn_api

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_config_stats(const moe_config* cfg, moe_stats_t* out) {
  TRY(validate(cfg));
  if (!out) return fail(MOE_ERR_INVALID_ARG, "null stats");
  compute_stats(*cfg, out);
  return MOE_OK;
}

int moe_create(const moe_config* cfg, const moe_weights* wts, void* stream, moe_handle** out) {
  (void)stream;
  TRY(validate(cfg));
  if (!wts || !out) return fail(MOE_ERR_INVALID_ARG, "null weights or output handle");
  *out = nullptr;
  const moe_config& c = *cfg;
  moe_weights host_w;
  std::vector<std::vector<char>> host_store;
  const moe_weights* w = wts;
  if (wts->on_device) {
    TRY(weights_to_host(c, wts, &host_w, host_store));
    w = &host_w;
  }
  const int P = c.act == MOE_ACT_SWIGLU ? 3 : 2;
  if (!w->W_grp) return fail(MOE_ERR_INVALID_ARG, "W_grp is required");
  if (c.K > 1 && !w->W_exp) return fail(MOE_ERR_INVALID_ARG, "W_exp is required when K > 1");
  for (int p = 0; p < P; ++p) {
    if (!w->base[p]) return fail(MOE_ERR_INVALID_ARG, "base[%d] is null", p);
    if (c.r > 0 && (!w->A[p] || !w->B[p])) return fail(MOE_ERR_INVALID_ARG, "A[%d]/B[%d] null with r > 0", p, p);
  }
  std::unique_ptr<moe_handle> h(new moe_handle());
  h->cfg = c;
  h->E = c.G * c.K;
  h->k = c.top_groups * c.top_experts;
  h->P = P;
  h->P_in = P - 1;
  h->mma = c.base_dtype;
  h->NU = c.r > 0 ? (int)roundup((long)c.K * h->P_in * RPAD, 64) : 0;
  h->NV = c.r > 0 ? (int)roundup((long)c.K * RPAD, 64) : 0;
  if (hipGetDevice(&h->device) != hipSuccess) return fail(MOE_ERR_HIP, "no HIP device");
  {
    // set-up of the no-allocation entry point on this device
    char* sp = nullptr;
    TRY(scratch_for_device(h->device, &sp));
  }
  {
    const char* names[3] = {"U", "G1", "G2"};
    for (int i = 0; i < 3; ++i) {
      char key[32];
      std::snprintf(key, sizeof(key), "CEFN_BM_%s", names[i]);
      if (const char* v = std::getenv(key)) h->bm_env[i] = std::atoi(v);
    }
    if (const char* v = std::getenv("CEFN_KS_G2")) h->ks_env = std::atoi(v);
    if (const char* v = std::getenv("CEFN_G2K")) h->g2k_env = std::atoi(v);
    if (const char* v = std::getenv("CEFN_G1K")) h->g1k_env = std::atoi(v);
    if (const char* v = std::getenv("CEFN_UT")) h->ut_env = std::atoi(v);
    if (const char* v = std::getenv("CEFN_GSORT")) h->gsort_env = std::atoi(v);
    if (const char* v = std::getenv("CEFN_TAIL_SLOTS")) h->tail_env = std::atoi(v);
  }

  // router weights and biases
  {
    // one score matrix for both levels: [W_grp | W_exp^0 | ... | W_exp^{G-1}],
    // sixteen k of a column contiguous (the order the score kernel reads)
    const int NC = c.G + (c.K > 1 ? c.G * c.K : 0);
    h->NCp = (int)roundup(NC, 32);
    std::vector<float> wr((size_t)c.d * h->NCp, 0.f);
    for (int k = 0; k < c.d; ++k)
      for (int col = 0; col < NC; ++col) {
        float v;
        if (col < c.G) {
          v = w->W_grp[(size_t)k * c.G + col];
        } else {
          const int g = (col - c.G) / c.K, j = (col - c.G) % c.K;
          v = w->W_exp[((size_t)g * c.d + k) * c.K + j];
        }
        wr[((size_t)(k / 16) * h->NCp + col) * 16 + (k % 16)] = v;
      }
    TRY(upload(h.get(), &h->Wr, wr));
    if (c.x_dtype != MOE_F32) {
      // three bf16 parts, each the nearest bf16 to what the previous parts
      // leave (every subtraction exact in fp32)
      const size_t n = wr.size();
      std::vector<uint16_t> wb(3 * n);
      for (size_t i = 0; i < n; ++i) {
        float rest = wr[i];
        for (int p = 0; p < 3; ++p) {
          const uint16_t b = host_f32_to_bf16(rest);
          uint32_t u = static_cast<uint32_t>(b) << 16;
          float bv;
          std::memcpy(&bv, &u, 4);
          wb[p * n + i] = b;
          rest -= bv;
        }
      }
      TRY(upload(h.get(), &h->Wb, wb));
    }
    if (w->group_bias) {
      std::vector<float> gb(w->group_bias, w->group_bias + c.G);
      TRY(upload(h.get(), &h->gbias, gb));
    }
    if (w->expert_bias && c.K > 1) {
      std::vector<float> eb(w->expert_bias, w->expert_bias + h->E);
      TRY(upload(h.get(), &h->ebias, eb));
    }
  }
  int rc = (h->mma == MOE_F32) ? build_weights<float>(h.get(), w) : build_weights<uint16_t>(h.get(), w);
  if (rc) {
    moe_destroy(h.release());
    return rc;
  }

  // workspace, one buffer carved for T_max tokens
  h->nt1 = (h->P_in * c.f + 255) / 256;
  {
    char* buf = nullptr;
    rc = dalloc(h.get(), &buf, carve_workspace(h.get(), c.T_max, nullptr, &h->ws));
    if (rc) {
      moe_destroy(h.release());
      return rc;
    }
    carve_workspace(h.get(), c.T_max, buf, &h->ws);
  }
  if (hipMemset(h->ws.cc, 0, sizeof(int) * ((size_t)h->ws.cc_n + 1)) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    moe_destroy(h.release());
    return fail(MOE_ERR_HIP, "initialising the workspace failed");
  }
  *out = h.release();
  return MOE_OK;
}

int moe_destroy(moe_handle* h) {
  if (!h) return MOE_OK;
  (void)hipDeviceSynchronize();
  for (void* p : h->allocs) (void)hipFree(p);
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  delete_bwd(h);
  delete_offload(h);
  delete h;
  return MOE_OK;
}

int moe_route(moe_handle* h, const void* X, int32_t T, const moe_route_out* out, void* stream) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  if (T < 0 || T > h->cfg.T_max) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, T_max=%d]", T, h->cfg.T_max);
  if (T > 0 && !X) return fail(MOE_ERR_INVALID_ARG, "null X");
  hipStream_t st = static_cast<hipStream_t>(stream);
  Prof pf{h, st, -1};
  if (h->prof && h->prof_calls < h->prof_max) pf.call = h->prof_calls++;
  RouteLive live{};
  TRY(run_route(h, h->ws, X, T, out, true, st, pf, live));
  hipError_t e = launch_zero(h->ws.cc, h->ws.cc_n, st);
  if (e != hipSuccess) return hip_fail(h, e, "clear counters");
  return MOE_OK;
}

}  // extern "C"

namespace cefn_api {

FactorLoc locate_factor(const moe_handle* h, int proj, int which, int expert) {
  const moe_config& c = h->cfg;
  int di, dn;
  dims(c, proj, di, dn);
  FactorLoc L{};
  L.n = which == 0 ? di : dn;
  const int K = c.K, g = expert / K, j = expert % K, nfb = c.f / 32;
  const bool int4 = c.resid == MOE_RESID_INT4_G32;
  const bool down = proj == h->P - 1;
  if (which == 0 && !down) {  // At
    L.kind = 0;
    L.src = h->At;
    L.sc = h->At_s;
    L.base = int4 ? g * h->at_gs : g * h->at_gs / 8;
    L.sbase = g * h->at_sgs;
    L.aux0 = (j * h->P_in + proj) * RPAD;
    L.aux1 = c.d / 16;
  } else if (which == 1 && !down) {  // B1
    L.kind = 1;
    L.src = h->B1;
    L.sc = h->B1_s;
    L.base = (long)(expert * h->P_in + proj) * nfb * 64;
    L.sbase = (long)(expert * h->P_in + proj) * nfb * RPAD;
    L.aux0 = 0;
    L.aux1 = 1;
  } else if (which == 0 && down) {  // Ad
    L.kind = 2;
    L.src = h->Ad;
    L.sc = h->Ad_s;
    L.base = (long)expert * nfb * 2 * 64;
    L.sbase = (long)expert * nfb * RPAD;
  } else {  // Bd
    L.kind = 3;
    L.src = h->Bd;
    L.sc = h->Bd_s;
    L.base = int4 ? g * h->bd_gs : g * h->bd_gs / 8;
    L.sbase = (long)expert * (c.d / 32) * RPAD;
    L.aux0 = j;
    L.aux1 = h->NV / 16;
  }
  return L;
}

// Routing, the optional per-group row sort and the activation conversion.
int fwd_prelude(moe_handle* h, Workspace& ws, const void* X, int T, const moe_route_out* routing, hipStream_t st,
                FwdState& fs) {
  const moe_config& c = h->cfg;
  fs.pf = Prof{h, st, -1};
  if (h->prof && h->prof_calls < h->prof_max) fs.pf.call = h->prof_calls++;
  Prof& pf = fs.pf;
  RouteLive& live = fs.live;
  TRY(run_route(h, ws, X, T, routing, routing != nullptr, st, pf, live));

  const int kg = c.top_groups;
  const int rows = T * kg;
  // With residuals the input projection's epilogue takes one step per expert
  // present in a 32-row block.  Sorting each group's rows by expert set
  // (the internal row map only; the routing outputs keep token order) makes
  // blocks purer than the per-tile sort can when there are many sets (8 or
  // more experts per group) and many rows (64 or more per group on
  // average); measured: large INT4 layer gemm1 395 -> 355 us, while on the
  // 4-expert fp16 layer the tile sort already suffices.
  const int* garow = ws.garow;
  const bool gsorted =
      ws.garow_sorted && (h->gsort_env == 1 || (h->gsort_env != 0 && c.K >= 8 && rows >= 64L * c.G));
  if (gsorted) {
    GroupSortArgs gs{ws.garow, ws.garow_sorted, live.goffsets, live.idx, c.G, c.K, kg, c.top_experts, h->k};
    hipError_t es = launch_group_sort(gs, rows, st);
    if (es != hipSuccess) return hip_fail(h, es, "group sort launch");
    garow = ws.garow_sorted;
  }
  fs.garow = garow;
  fs.gsorted = gsorted;
  // bf16 activations with fp16 MFMAs: the row GEMMs read an fp16 copy made
  // in one pass, instead of converting every staged row in their loaders
  fs.xg = X;
  fs.xt = c.x_dtype;
  if (ws.X16) {
    hipError_t e = launch_cvt_x(X, ws.X16, (long)T * c.d, st);
    if (e != hipSuccess) return hip_fail(h, e, "activation conversion launch");
    fs.xg = ws.X16;
    fs.xt = MOE_F16;
  }
  fs.splits = 1;
  return MOE_OK;
}

// The grouped GEMMs over the groups whose count in gcounts is non-zero,
// weights of group g at slot gslot[g] of the weight arrays (gslot null: g).
int fwd_gemms(moe_handle* h, Workspace& ws, const void* X, int T, void* Y, hipStream_t st, FwdState& fs,
              const int* gcounts, const int* gslot) {
  const moe_config& c = h->cfg;
  const int kg = c.top_groups;
  const int rows = T * kg;
  Prof& pf = fs.pf;
  RouteLive& live = fs.live;
  const int* garow = fs.garow;
  const bool gsorted = fs.gsorted;
  GemmArgs ga{};
  ga.gcounts = gcounts;
  ga.gslot = gslot;
  ga.goffsets = live.goffsets;
  ga.G = c.G;
  ga.K = c.K;
  ga.kg = kg;
  ga.ke = c.top_experts;
  ga.k = h->k;
  ga.resid = c.resid;
  ga.act = c.act == MOE_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU;
  ga.X = X;
  ga.d = c.d;
  ga.f = c.f;
  ga.garow = garow;
  ga.rows_sorted = gsorted ? 1 : 0;
  ga.idx = live.idx;
  ga.w = live.w;
  ga.U = ws.U;
  ga.NU = h->NU;
  ga.V = ws.V;
  ga.NV = h->NV;
  ga.Vp = ws.Vp;
  ga.vp_rows = ws.T_cap * kg;
  ga.H = ws.H;
  ga.ypart = ws.ypart;
  ga.Y = Y;
  ga.ksplit = 1;
  ga.rows_total = (long)rows;
  int splits = 1;
  bool g1k = false, g1k2 = false;  // gemm1 ran with the k-split tiles (d in four, in two)
  hipError_t e;
  const void* xg = fs.xg;
  const int xt = fs.xt;
  if (c.r > 0) {
    GemmArgs u = ga;
    u.X = xg;
    u.Bw = h->At;
    u.bw_gstride = h->at_gs;
    u.bw_scale = h->At_s;
    u.bws_gstride = h->at_sgs;
    // many rows: the tile engine over 64- or 128-row x 256-column tiles
    // once there are a chip's worth of them (each row of X read once per 256
    // columns of U); otherwise 32-row tiles with d split over the wavefronts
    const int nut = (h->NU + 255) / 256;
    // 128 rows halve the INT4 decode per row and measured faster than 64
    // rows even with half the compute units busy
    int ubm = (long)max_mtiles(T, kg, c.G, 128) * nut >= 128 ? 128 : 64;
    if (h->bm_env[GK_U] >= 64) ubm = h->bm_env[GK_U];
    const bool ut = h->ut_env == 1 || (h->ut_env != 0 && (long)max_mtiles(T, kg, c.G, 64) * nut >= 256);
    pf.begin(2);
    if (ut)
      e = launch_gemm(GK_UT, xt, h->mma, h->mma == MOE_F32 ? 64 : ubm, u,
                      max_mtiles(T, kg, c.G, h->mma == MOE_F32 ? 64 : ubm), nut, 1, st);
    else
      e = launch_gemm(GK_U, xt, h->mma, 32, u, max_mtiles(T, kg, c.G, 32), 1, 1, st);
    if (e != hipSuccess) return hip_fail(h, e, "ugemm launch");
    pf.end(2);
  }
  {
    GemmArgs g1 = ga;
    g1.X = xg;
    g1.Bw = h->W1;
    g1.bw_gstride = h->w1_gs;
    g1.B1 = h->B1;
    g1.b1_scale = h->B1_s;
    g1.Ad = h->Ad;
    g1.ad_scale = h->Ad_s;
    const int nt = (h->P_in * c.f + 255) / 256;
    const int bm = pick_bm(h, GK_G1, rows, nt, 1);
    // few tiles: 32-row tiles with d split over the wavefronts.  Under half
    // a round of 256-column tiles at 32 rows: 64-column tiles, d in four
    // (tiny layers gain: fp32 layer 29 -> 18 us).  128-column tiles with d
    // in two (CEFN_G1K=2) are never picked: on the decode layer (about
    // 132 tiles of 256 columns) they measured 93 us against 75 us, the
    // four-part tiles 80 us.
    const bool k_ok = c.r == 0 || ws.nt1k > 0;
    const bool auto_k = h->g1k_env < 0 && h->bm_env[GK_G1] == 0 && bm == 32;
    g1k = k_ok && (h->g1k_env == 1 || (auto_k && (long)max_mtiles(T, kg, c.G, 32) * nt < 128));
    g1k2 = !g1k && k_ok && h->g1k_env == 2;
    pf.begin(3);
    if (g1k)
      e = launch_gemm(GK_G1K, xt, h->mma, 32, g1, max_mtiles(T, kg, c.G, 32), h->P_in * c.f / 64, 1, st);
    else if (g1k2)
      e = launch_gemm(GK_G1K2, xt, h->mma, 32, g1, max_mtiles(T, kg, c.G, 32), (h->P_in * c.f + 127) / 128, 1,
                      st);
    else
      e = launch_gemm(GK_G1, xt, h->mma, bm, g1, max_mtiles(T, kg, c.G, bm), nt, 1, st);
    if (e != hipSuccess) return hip_fail(h, e, "gemm1 launch");
    pf.end(3);
  }
  if (c.r > 0) {
    VReduceArgs va{};
    va.Vp = ws.Vp;
    va.V = ws.V;
    va.garow = garow;
    va.gidx = live.gidx;
    va.idx = live.idx;
    va.vp_rows = ws.T_cap * kg;
    va.rows = rows;
    va.ntiles = g1k ? ws.nt1k : g1k2 ? (h->P_in * c.f + 127) / 128 : h->nt1;
    va.NV = h->NV;
    va.K = c.K;
    va.kg = kg;
    va.ke = c.top_experts;
    va.k = h->k;
    pf.begin(4);
    e = launch_vreduce(h->mma, va, st);
    if (e != hipSuccess) return hip_fail(h, e, "vreduce launch");
    pf.end(4);
  }
  {
    GemmArgs g2 = ga;
    g2.Bw = h->W2;
    g2.bw_gstride = h->w2_gs;
    g2.Bd = h->Bd;
    g2.bd_gstride = h->bd_gs;
    g2.bd_scale = h->Bd_s;
    g2.zero_ptr = ws.cc;
    g2.zero_n = ws.cc_n;
    const int nt = (c.d + 255) / 256;
    // 256-column tiles with the rows staged through LDS and the k range split
    // over workgroups; the variant that splits f inside each workgroup over
    // 64 x 128 tiles is kept as an option (CEFN_G2K=1)
    const bool ksplit_wg = h->g2k_env > 0;
    pf.begin(5);
    if (ksplit_wg) {
      splits = 1;
      e = launch_gemm(GK_G2K, c.x_dtype, h->mma, 64, g2, max_mtiles(T, kg, c.G, 64), 1, 1, st);
    } else {
      int bm = 128;
      pick_g2(h, rows, nt, bm, splits);
      g2.ksplit = splits;
      // Last-round split: with one k split, a last round of tiles that
      // would leave most compute units idle is cut along k (the first piece
      // writes fp32 partials, the others land in the unused split slices of
      // ypart, and a small kernel adds them into the partials or Y).  Round
      // size: 256 compute units x two resident 128-row tiles of 16-bit types
      // (one 256-row tile); shorter tiles are left alone.
      int slots = (h->mma != MOE_F32 && bm >= 128) ? (bm == 128 ? 512 : 256) : 0;
      if (h->tail_env >= 0) slots = h->tail_env;
      const long room = ((long)kMaxSplits * ws.T_cap * kg - rows) * c.d;  // floats after slice 0
      if (splits == 1 && slots > 0 && room >= (long)bm * 256) {
        g2.tail_slots = slots;
        g2.tail_smax = 8;
        g2.tail_max_pieces = (int)std::min<long>(room / ((long)bm * 256), 1L << 20);
        g2.tailpart = ws.ypart + (long)rows * c.d;
        // whole tiles plus at most one round of pieces
        e = launch_gemm(GK_G2, c.x_dtype, h->mma, bm, g2, max_mtiles(T, kg, c.G, bm) * nt + slots, 1, 1, st);
        if (e == hipSuccess) e = launch_tailfix(c.x_dtype, bm, g2, st);
      } else {
        e = launch_gemm(GK_G2, c.x_dtype, h->mma, bm, g2, max_mtiles(T, kg, c.G, bm), nt, splits, st);
      }
    }
    if (e != hipSuccess) return hip_fail(h, e, "gemm2 launch");
    pf.end(5);
  }
  fs.splits = splits;
  return MOE_OK;
}

// Sum over chosen groups and k splits (when the down projection left partials).
int fwd_combine(moe_handle* h, Workspace& ws, int T, void* Y, hipStream_t st, FwdState& fs) {
  const moe_config& c = h->cfg;
  const int kg = c.top_groups, splits = fs.splits;
  if (kg > 1 || splits > 1) {
    CombineArgs ca{ws.ypart, Y, T, c.d, kg, splits};
    fs.pf.begin(6);
    hipError_t e = launch_combine(c.x_dtype, ca, st);
    if (e != hipSuccess) return hip_fail(h, e, "combine launch");
    fs.pf.end(6);
  }
  return MOE_OK;
}

// The whole layer on workspace ws (T >= 1, arguments checked by the caller).
// The last GEMM clears ws's counters again for the next pass.
int forward_impl(moe_handle* h, Workspace& ws, const void* X, int T, void* Y, const moe_route_out* routing,
                 hipStream_t st) {
  FwdState fs{};
  TRY(fwd_prelude(h, ws, X, T, routing, st, fs));
  TRY(fwd_gemms(h, ws, X, T, Y, st, fs, fs.live.gcounts, nullptr));
  return fwd_combine(h, ws, T, Y, st, fs);
}

}  // namespace cefn_api

extern "C" {

int moe_forward(moe_handle* h, const void* X, int32_t T, void* Y, const moe_route_out* routing,
                void* stream) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  const moe_config& c = h->cfg;
  if (T < 0 || T > c.T_max) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, T_max=%d]", T, c.T_max);
  // no tokens: nothing to compute, but the routing outputs still say so
  if (T == 0) return routing ? moe_route(h, X, 0, routing, stream) : MOE_OK;
  if (!X || !Y) return fail(MOE_ERR_INVALID_ARG, "null X or Y");
  if (X == Y) return fail(MOE_ERR_INVALID_ARG, "X and Y may not alias");
  if (h->off) return fail(MOE_ERR_UNSUPPORTED, "the handle's groups are offloaded: use moe_forward_offload");
  return forward_impl(h, h->ws, X, T, Y, routing, static_cast<hipStream_t>(stream));
}

int moe_forward_noalloc(moe_handle* h, const void* X, int32_t T, void* Y, const moe_route_out* routing,
                        void* stream) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  const moe_config& c = h->cfg;
  if (T < 0 || T > c.T_max) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, T_max=%d]", T, c.T_max);
  if (T == 0) return routing ? moe_route(h, X, 0, routing, stream) : MOE_OK;
  if (!X || !Y) return fail(MOE_ERR_INVALID_ARG, "null X or Y");
  if (X == Y) return fail(MOE_ERR_INVALID_ARG, "X and Y may not alias");
  if (h->off) return fail(MOE_ERR_UNSUPPORTED, "the handle's groups are offloaded: use moe_forward_offload");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "no HIP device");
  if (dev != h->device) return fail(MOE_ERR_INVALID_ARG, "handle lives on device %d, device %d is current", h->device, dev);
  char* base = nullptr;
  TRY(scratch_for_device(dev, &base));
  Workspace ws;
  const size_t need = carve_workspace(h, T, nullptr, &ws);
  if (need > kScratchBytes)
    return fail(MOE_ERR_INVALID_ARG, "T=%d needs %zu bytes of workspace, more than the %zu of the static scratch",
                T, need, kScratchBytes);
  carve_workspace(h, T, base, &ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the array keeps whatever the last call left: the counters must start at zero
  const hipError_t e = launch_zero(ws.cc, ws.cc_n, st);
  if (e != hipSuccess) return hip_fail(h, e, "clear counters");
  return forward_impl(h, ws, X, T, Y, routing, st);
}


int moe_debug_residual(moe_handle* h, int32_t proj, int32_t which, int32_t expert, float* values,
                       int8_t* q, uint16_t* scale_bits) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  const moe_config& c = h->cfg;
  if (c.r == 0) return fail(MOE_ERR_INVALID_ARG, "layer has no residual");
  if (proj < 0 || proj >= h->P || (which != 0 && which != 1) || expert < 0 || expert >= h->E || !values)
    return fail(MOE_ERR_INVALID_ARG, "bad residual selector");
  FactorLoc L = locate_factor(h, proj, which, expert);
  const int n = L.n, r = c.r;
  const bool int4 = c.resid == MOE_RESID_INT4_G32;
  const int kind = L.kind, aux0 = L.aux0;
  const long sbase = L.sbase;
  const uint16_t* sc = L.sc;
  float* dout = nullptr;
  if (hipMalloc(&dout, sizeof(float) * (size_t)n * r) != hipSuccess) return fail(MOE_ERR_OOM, "debug buffer");
  hipError_t e = launch_debug_decode(h->mma, c.resid, kind, L.src, sc, L.base, sbase, n, r, aux0, L.aux1, dout, r,
                                     nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(values, dout, sizeof(float) * (size_t)n * r, hipMemcpyDeviceToHost);
  (void)hipFree(dout);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "debug decode: %s", hipGetErrorString(e));
  if (int4 && (q || scale_bits)) {
    // codes and scales follow from the decoded values and the stored scales
    std::vector<uint16_t> sc_host;
    const long ns = (long)(n / 32) * r;
    sc_host.resize(ns);
    for (int b = 0; b < n / 32; ++b)
      for (int rho = 0; rho < r; ++rho) {
        long off;
        if (kind == 0) {
          const int ncol = aux0 + rho;
          off = sbase + ((long)(ncol / 32) * (c.d / 32) + b) * 32 + (ncol % 32);
        } else {
          off = sbase + (long)b * RPAD + rho;
        }
        if (hipMemcpy(&sc_host[(size_t)b * r + rho], sc + off, 2, hipMemcpyDeviceToHost) != hipSuccess)
          return fail(MOE_ERR_HIP, "debug scale read");
      }
    if (scale_bits) std::memcpy(scale_bits, sc_host.data(), ns * 2);
    if (q) {
      for (int i = 0; i < n; ++i)
        for (int rho = 0; rho < r; ++rho) {
          const float s = host_f16_to_f32(sc_host[(size_t)(i / 32) * r + rho]);
          const float v = values[(size_t)i * r + rho];
          q[(size_t)i * r + rho] = s > 0.f ? static_cast<int8_t>(v / s) : 0;
        }
    }
  }
  return MOE_OK;
}

int moe_stats(const moe_handle* h, moe_stats_t* out) {
  if (!h || !out) return fail(MOE_ERR_INVALID_ARG, "null handle or stats");
  compute_stats(h->cfg, out);
  return MOE_OK;
}

int moe_debug_dequant(moe_handle* h, int32_t proj, int32_t which, int32_t expert, float* host_out) {
  return moe_debug_residual(h, proj, which, expert, host_out, nullptr, nullptr);
}

int moe_debug_q(moe_handle* h, int32_t proj, int32_t which, int32_t expert, int8_t* q, uint16_t* scale_bits) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  if (h->cfg.resid != MOE_RESID_INT4_G32) return fail(MOE_ERR_INVALID_ARG, "layer residual is not INT4");
  if (proj < 0 || proj >= h->P) return fail(MOE_ERR_INVALID_ARG, "bad residual selector");
  int di, dn;
  dims(h->cfg, proj, di, dn);
  std::vector<float> vals((size_t)(which == 0 ? di : dn) * h->cfg.r);
  return moe_debug_residual(h, proj, which, expert, vals.data(), q, scale_bits);
}

int moe_profile_begin(moe_handle* h, int32_t max_calls, int32_t stage_mask) {
  if (!h || max_calls <= 0) return fail(MOE_ERR_INVALID_ARG, "bad profile request");
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  h->ev.assign((size_t)max_calls * kStages * 2, nullptr);
  for (auto& e : h->ev)
    if (hipEventCreate(&e) != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreate");
  h->ev_used.assign((size_t)max_calls * kStages, 0);
  h->prof = true;
  h->prof_mask = stage_mask;
  h->prof_max = max_calls;
  h->prof_calls = 0;
  return MOE_OK;
}

int moe_profile_end(moe_handle* h, float* stage_ms, int32_t n_stages_cap, int32_t* n_stages,
                    int32_t* n_calls, char* names, int32_t names_cap) {
  if (!h || !h->prof) return fail(MOE_ERR_INVALID_ARG, "profiling not active");
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_ERR_HIP, "synchronise");
  std::vector<float> tot(kStages, 0.f);
  for (int call = 0; call < h->prof_calls; ++call)
    for (int s = 0; s < kStages; ++s) {
      if (!h->ev_used[(size_t)call * kStages + s]) continue;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, h->ev[((size_t)call * kStages + s) * 2],
                              h->ev[((size_t)call * kStages + s) * 2 + 1]) == hipSuccess)
        tot[s] += ms;
    }
  if (stage_ms)
    for (int s = 0; s < std::min<int>(kStages, n_stages_cap); ++s) stage_ms[s] = tot[s];
  if (n_stages) *n_stages = kStages;
  if (n_calls) *n_calls = h->prof_calls;
  if (names && names_cap > 0) {
    std::string all;
    for (int s = 0; s < kStages; ++s) {
      if (s) all += ",";
      all += kStageNames[s];
    }
    std::snprintf(names, names_cap, "%s", all.c_str());
  }
  h->prof = false;
  return MOE_OK;
}

}  // extern "C"

