// Host-side weight preparation for moe_create: INT4 quantisation of the
// residual factors and re-layout of every weight into the fragment-major
// order the MFMA kernels read (see kernels.h for the layouts).
//
// INT4 rule ("Breaking the MoE LLM Trilemma", papernotes.org note, key
// design 4 stores the residual in INT4; block size, symmetry and rounding
// are this library's reading): per factor [n][r], blocks of 32 consecutive
// entries along n for each rank column; scale = fp16 round-to-nearest-even
// of amax / 7 (FP32 division); q = clamp(rint(v / scale), -8, 7) in FP32
// with ties to even; a zero scale gives q = 0.  Stored nibble = q + 8.
#include "pack.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace cefn {

uint16_t host_f32_to_f16(float v) {
  _Float16 h = static_cast<_Float16>(v);
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

float host_f16_to_f32(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

uint16_t host_f32_to_bf16(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

Q4 quantize_g32(const float* M, int n, int r) {
  Q4 out;
  out.n = n;
  out.r = r;
  out.q.assign((size_t)n * r, 0);
  out.s.assign((size_t)(n / 32) * r, 0);
  for (int b = 0; b < n / 32; ++b) {
    for (int c = 0; c < r; ++c) {
      float amax = 0.f;
      for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(M[(size_t)(b * 32 + i) * r + c]));
      const float ratio = amax / 7.0f;
      const uint16_t sb = host_f32_to_f16(ratio);
      const float s = host_f16_to_f32(sb);
      out.s[(size_t)b * r + c] = sb;
      for (int i = 0; i < 32; ++i) {
        int qi = 0;
        if (s > 0.f) {
          float t = std::nearbyint(M[(size_t)(b * 32 + i) * r + c] / s);
          t = std::min(std::max(t, -8.0f), 7.0f);
          qi = static_cast<int>(t);
        }
        out.q[(size_t)(b * 32 + i) * r + c] = static_cast<int8_t>(qi);
      }
    }
  }
  return out;
}

void parallel_for(int n, const std::function<void(int)>& fn) {
  unsigned hw = std::thread::hardware_concurrency();
  int nt = (int)std::min<unsigned>(hw ? hw : 1, 16);
  if (n < 2 || nt < 2) {
    for (int i = 0; i < n; ++i) fn(i);
    return;
  }
  nt = std::min(nt, n);
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int i = t; i < n; i += nt) fn(i);
    });
  for (auto& x : th) x.join();
}

}  // namespace cefn
