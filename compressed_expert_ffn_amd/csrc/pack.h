// Host-side helpers for weight preparation (quantisation, dtype bits,
// fragment-major writers).  Layouts are described in kernels.h.
#pragma once
#include <stdint.h>

#include <functional>
#include <vector>

namespace cefn {

struct Q4 {
  int n = 0, r = 0;
  std::vector<int8_t> q;    // [n][r]
  std::vector<uint16_t> s;  // [n/32][r] fp16 bits
  int code(int i, int c) const { return q[(size_t)i * r + c]; }
  uint16_t scale(int i, int c) const { return s[(size_t)(i / 32) * r + c]; }
};

uint16_t host_f32_to_f16(float v);
float host_f16_to_f32(uint16_t b);
uint16_t host_f32_to_bf16(float v);

Q4 quantize_g32(const float* M, int n, int r);

void parallel_for(int n, const std::function<void(int)>& fn);

// Record an error for moe_last_error() (printf-style) and return code.
int report_error(int code, const char* fmt, ...);

// Depth k held by element e of lane half h in k-step ks of a fragment-major
// matrix.  Permuted order (Kd a multiple of 64): inside every 64-deep block,
// lane half h covers 32 consecutive k across the block's 4 k-steps, so a
// lane's share of a 64-deep stage of a row-major activation is contiguous.
// Plain order: the 16-deep k-step is split in two halves of 8.
inline int frag_k(int ks, int h, int e, bool perm) {
  return perm ? 64 * (ks >> 2) + 32 * h + 8 * (ks & 3) + e : 16 * ks + 8 * h + e;
}

// Fragment-major write of an N x Kd matrix: get(n, k) -> T.
// dst holds (N/32) * (Kd/16) * 64 * 8 elements, element (n, k) at fragment
// (n/32) * (Kd/16) + ks, lane (n % 32) + 32 h, slot e with frag_k(ks, h, e) = k.
template <class T, class Get>
void pack_frag(T* dst, int N, int Kd, bool perm, Get get) {
  const int KS = Kd / 16;
  parallel_for(N / 32, [&](int nb) {
    for (int ks = 0; ks < KS; ++ks)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          const int n = nb * 32 + (lane & 31);
          const int k = frag_k(ks, lane >> 5, e, perm);
          dst[((size_t)(nb * KS + ks) * 64 + lane) * 8 + e] = get(n, k);
        }
  });
}

// Same order with 8 nibbles (q + 8) per 32-bit word: getq(n, k) -> q in [-8, 7].
template <class GetQ>
void pack_frag_int4(uint32_t* dst, int N, int Kd, bool perm, GetQ getq) {
  const int KS = Kd / 16;
  parallel_for(N / 32, [&](int nb) {
    for (int ks = 0; ks < KS; ++ks)
      for (int lane = 0; lane < 64; ++lane) {
        uint32_t word = 0;
        for (int e = 0; e < 8; ++e) {
          const int n = nb * 32 + (lane & 31);
          const int k = frag_k(ks, lane >> 5, e, perm);
          word |= static_cast<uint32_t>(getq(n, k) + 8) << (4 * e);
        }
        dst[(size_t)(nb * KS + ks) * 64 + lane] = word;
      }
  });
}

// A_down operand of the fused h . A_down product: for f-block fb (32 rows of
// A_down) and k-step s (0, 1), lane l holds column rho = l % 32 (zero for
// rho >= r) and, in slot e, row fb*32 + ad_row(s, l / 32, e) -- the rows a
// lane of the transposed accumulator holds for its token.
inline int ad_row(int s, int h, int e) { return 16 * s + 4 * h + (e < 4 ? e : e + 4); }

}  // namespace cefn
