// Shared device-side definitions: element types, MFMA fragments, the
// fragment-major weight layout, INT4 decoding and the workspace/argument
// structures the kernels exchange.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cefn {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum Resid : int { RS_NONE = 0, RS_F32 = 1, RS_F16 = 2, RS_INT4 = 3 };
enum Act : int { ACT_GELU = 0, ACT_SWIGLU = 1 };

constexpr int WAVE = 64;
constexpr int CHUNK = 256;     // assignments per counting chunk (one scatter block)
constexpr int MAX_SLOTS = 16;  // top_groups * top_experts
constexpr int MAX_KG = 8;
constexpr int RPAD = 16;       // residual rank padded to one 16-deep MFMA k-step

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile
// time (register arrays indexed by i stay in registers).
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// ---------------------------------------------------------------- scalars --
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {  // nearest, ties to even
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  _Float16 h = static_cast<_Float16>(v);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// element type of an activation/output buffer
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { using T = float; };
template <> struct Elem<DT_F16> { using T = uint16_t; };
template <> struct Elem<DT_BF16> { using T = uint16_t; };

template <int DT>
__device__ __forceinline__ float load_as_f32(const typename Elem<DT>::T* p, long i) {
  if constexpr (DT == DT_F32) return p[i];
  else if constexpr (DT == DT_F16) return f16_bits_to_f32(p[i]);
  else return bf16_bits_to_f32(p[i]);
}
template <int DT>
__device__ __forceinline__ typename Elem<DT>::T from_f32(float v) {
  if constexpr (DT == DT_F32) return v;
  else if constexpr (DT == DT_F16) return f32_to_f16_bits(v);
  else return f32_to_bf16_bits(v);
}

// -------------------------------------------------------------- fragments --
// An MFMA operand fragment is, per lane, 8 consecutive k values of one row
// (A) or one column (B).  For 16-bit types that is 16 bytes and feeds one
// v_mfma_*_32x32x16 / 16x16x32; for fp32 it is 32 bytes feeding eight
// v_mfma_f32_32x32x2 / 16x16x4 (lane half h takes k = 8h + i in step i, so
// both operands see the same k permutation).
template <int TY> struct Frag;
template <> struct Frag<DT_F16> { using T = h8; static constexpr int bytes = 16; };
template <> struct Frag<DT_BF16> { using T = b8; static constexpr int bytes = 16; };
template <> struct Frag<DT_F32> { using T = f8; static constexpr int bytes = 32; };

template <int TY>
__device__ __forceinline__ f16v mfma32(typename Frag<TY>::T a, typename Frag<TY>::T b, f16v c) {
  if constexpr (TY == DT_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  } else if constexpr (TY == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
    return c;
  }
}
template <int TY>
__device__ __forceinline__ f4v mfma16(typename Frag<TY>::T a, typename Frag<TY>::T b, f4v c) {
  if constexpr (TY == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  } else if constexpr (TY == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
  }
}

// Row of element v (0..15) of a 32x32 accumulator held by lane l; its column
// is l % 32.
__device__ __forceinline__ int acc32_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
// Row of element v (0..3) of a 16x16 accumulator; column l % 16.
__device__ __forceinline__ int acc16_row(int v, int lane) { return 4 * (lane >> 4) + v; }

// Convert 8 floats to a fragment of type TY.
template <int TY>
__device__ __forceinline__ typename Frag<TY>::T to_frag(const float* v) {
  typename Frag<TY>::T r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (TY == DT_F16) r[i] = static_cast<_Float16>(v[i]);
    else if constexpr (TY == DT_BF16) r[i] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(v[i]));
    else r[i] = v[i];
  }
  return r;
}

template <int TY>
__device__ __forceinline__ typename Frag<TY>::T zero_frag() {
  typename Frag<TY>::T r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = 0;
  return r;
}

// Load a fragment stored in type TY (16 or 32 contiguous bytes).
template <int TY>
__device__ __forceinline__ typename Frag<TY>::T load_frag(const void* p) {
  if constexpr (TY == DT_F32) {
    const f4v* q = reinterpret_cast<const f4v*>(p);
    f4v a = q[0], b = q[1];
    f8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
  } else {
    u4v u = *reinterpret_cast<const u4v*>(p);
    return __builtin_bit_cast(typename Frag<TY>::T, u);
  }
}

// INT4 decode: nibble e (bits 4e..4e+3 of the 32-bit word) holds q + 8.
// The decoded value (float)q * scale is exact in fp32.
__device__ __forceinline__ float int4_value(uint32_t word, int e, float scale) {
  int nib = static_cast<int>((word >> (4 * e)) & 15u);
  return static_cast<float>(nib - 8) * scale;
}

// fp16 fragments decode with packed fp16 arithmetic: byte permutes put
// codes 2i and 2i+1 in the two halves of dword i (fragment order); a code c
// (= q + 8) placed in the low mantissa bits of the fp16 1024.0 is the fp16
// number 1024 + c, subtracting 1032 leaves q exactly, and one fp16 multiply
// by the scale pair rounds the exact product q * scale once -- the same
// value as the (exact) fp32 product converted to fp16.
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h8 int4_frag_f16_pairs(uint32_t word, u4v sc) {
  const uint32_t odd = word >> 4;
  u4v d;
  // bytes of {word, odd}: word byte b holds codes 2b, 2b+1; odd byte b holds
  // code 2b+1 in its low nibble; selector 0x0c gives a zero byte
  d[0] = __builtin_amdgcn_perm(word, odd, 0x0c000c04u);
  d[1] = __builtin_amdgcn_perm(word, odd, 0x0c010c05u);
  d[2] = __builtin_amdgcn_perm(word, odd, 0x0c020c06u);
  d[3] = __builtin_amdgcn_perm(word, odd, 0x0c030c07u);
  const h2v off = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  u4v r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // (vector elements go through plain scalars: a bit cast applied
    // directly to an element of a vector read element 0 in this compiler)
    const uint32_t code = (d[i] & 0x000F000Fu) | 0x64006400u;
    const uint32_t scale = sc[i];
    const h2v q = __builtin_bit_cast(h2v, code) - off;
    const h2v p = q * __builtin_bit_cast(h2v, scale);
    r[i] = __builtin_bit_cast(uint32_t, p);
  }
  return __builtin_bit_cast(h8, r);
}

// Decode 8 INT4 codes that share one scale (fp16 bits).
template <int TY>
__device__ __forceinline__ typename Frag<TY>::T int4_frag_1scale(uint32_t word, uint16_t scale_bits) {
  if constexpr (TY == DT_F16) {
    const uint32_t p = static_cast<uint32_t>(scale_bits) * 0x00010001u;
    const u4v sc = {p, p, p, p};
    return int4_frag_f16_pairs(word, sc);
  } else {
    const float scale = f16_bits_to_f32(scale_bits);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = int4_value(word, e, scale);
    return to_frag<TY>(v);
  }
}
// Decode 8 INT4 codes with one scale each (8 consecutive fp16 scales held
// in a 16-byte vector).
template <int TY>
__device__ __forceinline__ typename Frag<TY>::T int4_frag_8scale(uint32_t word, u4v s) {
  if constexpr (TY == DT_F16) {
    return int4_frag_f16_pairs(word, s);
  } else {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t bits = static_cast<uint16_t>((s[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      v[e] = int4_value(word, e, f16_bits_to_f32(bits));
    }
    return to_frag<TY>(v);
  }
}

// Position of the 8-bit word g in the binary reflected Gray code sequence
// (prefix XOR from the top bit down).  Among words with the same number of
// set bits, consecutive ones in that order differ by moving one bit, so
// rows sorted by the rank of their expert set see, within a block of
// neighbours, sets that differ by one expert.
__device__ __forceinline__ uint32_t gray_rank8(uint32_t g) {
  g ^= g >> 1;
  g ^= g >> 2;
  g ^= g >> 4;
  return g & 255u;
}

// ----------------------------------------------------------- fast math ---
// SiLU z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp
// each) instead of an IEEE division sequence.
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
__device__ __forceinline__ float gelu_tanh_f(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float u = c * (z + 0.044715f * z * z * z);
  return 0.5f * z * (1.0f + tanhf(u));
}

}  // namespace cefn
