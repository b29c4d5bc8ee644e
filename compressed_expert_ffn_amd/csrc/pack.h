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

// Fragment-major write of an N x Kd matrix: get(n, k) -> T.
// dst holds (N/32) * (Kd/16) * 64 * 8 elements.
template <class T, class Get>
void pack_frag(T* dst, int N, int Kd, Get get) {
  const int KS = Kd / 16;
  parallel_for(N / 32, [&](int nb) {
    for (int ks = 0; ks < KS; ++ks)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          const int n = nb * 32 + (lane & 31);
          const int k = ks * 16 + 8 * (lane >> 5) + e;
          dst[((size_t)(nb * KS + ks) * 64 + lane) * 8 + e] = get(n, k);
        }
  });
}

// Same order with 8 nibbles (q + 8) per 32-bit word: getq(n, k) -> q in [-8, 7].
template <class GetQ>
void pack_frag_int4(uint32_t* dst, int N, int Kd, GetQ getq) {
  const int KS = Kd / 16;
  parallel_for(N / 32, [&](int nb) {
    for (int ks = 0; ks < KS; ++ks)
      for (int lane = 0; lane < 64; ++lane) {
        uint32_t word = 0;
        for (int e = 0; e < 8; ++e) {
          const int n = nb * 32 + (lane & 31);
          const int k = ks * 16 + 8 * (lane >> 5) + e;
          word |= static_cast<uint32_t>(getq(n, k) + 8) << (4 * e);
        }
        dst[(size_t)(nb * KS + ks) * 64 + lane] = word;
      }
  });
}

}  // namespace cefn
