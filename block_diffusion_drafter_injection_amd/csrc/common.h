// Device-side helpers shared by the libdflash kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16-byte register payload
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxQkLayers = 16;   // layers whose QK-norm key gains one injection launch carries

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float32 -> bfloat16 with round-to-nearest-even: gfx950's v_cvt_pk_bf16_f32
// (the default rounding mode is nearest-even; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
// Two values rounded at once, packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Two-term bfloat16 split: x ~= hi + lo with |x - hi - lo| <= 2^-16 |x|.
__device__ __forceinline__ void split_hilo(float x, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}
// The same for a pair, results packed as two bf16 per word.
__device__ __forceinline__ void split_hilo2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Eight values -> (hi, lo) operand fragments of one MFMA input (8 bf16 each).
__device__ __forceinline__ void split_hilo8(const float* x, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) split_hilo2(x[2 * k], x[2 * k + 1], h[k], l[k]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Where an activation producer writes its result, in the form its consumer reads.
enum ActMode : int { ACT_F32 = 0, ACT_HILO = 1, ACT_BF16 = 2 };
struct ActOut {
  void* p0;   // F32: float plane; HILO: hi plane; BF16: the plane
  void* p1;   // HILO: lo plane
  int ld;     // row stride in elements
  int mode;
};
struct ActIn {
  const void* p0;
  const void* p1;
  int ld;
  int mode;
  const int* rows;   // optional gather: logical row r reads source row rows[r] (device)
};

__device__ __forceinline__ void act_store(const ActOut& o, int row, int col, float v) {
  size_t i = (size_t)row * o.ld + col;
  if (o.mode == ACT_F32) {
    ((float*)o.p0)[i] = v;
  } else if (o.mode == ACT_HILO) {
    bf16_t h, l;
    split_hilo(v, h, l);
    ((bf16_t*)o.p0)[i] = h;
    ((bf16_t*)o.p1)[i] = l;
  } else {
    ((bf16_t*)o.p0)[i] = f2bf(v);
  }
}

// Four consecutive columns (col % 4 == 0, ld % 4 == 0).
__device__ __forceinline__ void act_store4(const ActOut& o, int row, int col, float4 v) {
  size_t i = (size_t)row * o.ld + col;
  if (o.mode == ACT_F32) {
    *(float4*)((float*)o.p0 + i) = v;
  } else if (o.mode == ACT_HILO) {
    uint2 hv, lv;
    split_hilo2(v.x, v.y, hv.x, lv.x);
    split_hilo2(v.z, v.w, hv.y, lv.y);
    *(uint2*)((bf16_t*)o.p0 + i) = hv;
    *(uint2*)((bf16_t*)o.p1 + i) = lv;
  } else {
    uint2 hv;
    hv.x = pack_bf16x2(v.x, v.y);
    hv.y = pack_bf16x2(v.z, v.w);
    *(uint2*)((bf16_t*)o.p0 + i) = hv;
  }
}

template <typename T> __device__ __forceinline__ float ld_f(const T* p, size_t i);
template <> __device__ __forceinline__ float ld_f<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_f<bf16_t>(const bf16_t* p, size_t i) { return bf2f(p[i]); }

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64-bit
// multiplies, key advanced by the two Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Standard Gumbel noise G = -ln(-ln u) from one 32-bit word, u = ((x>>8)+0.5)/2^24.
// y + 0.5 needs 25 significant bits when y >= 2^23, so u is not formed there;
// instead -ln u = -log1p(-(2^24-1-y+0.5)/2^24), whose argument is exact in
// float32.  Both branches evaluate -ln u from an exactly represented input.
__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
  const uint32_t y = x >> 8;
  float t;
  if (y >= (1u << 23)) {
    const float w = ((float)(16777215u - y) + 0.5f) * (1.0f / 16777216.0f);
    t = -log1pf(-w);
  } else {
    t = -logf(((float)y + 0.5f) * (1.0f / 16777216.0f));
  }
  return -logf(t);
}

}  // namespace dflash
