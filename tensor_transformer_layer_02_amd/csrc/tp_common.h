// Shared device-side definitions of the gfx950 kernels: storage types,
// bf16 rounding, GeLU, MFMA vector types and launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

typedef uint16_t bf16_t;  // bfloat16 storage (raw bits)
struct f16_t {            // IEEE half storage (raw bits; a distinct type so templates can tell it apart)
    uint16_t bits;
};
static_assert(sizeof(f16_t) == 2, "f16_t is two bytes");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw;

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 in the default
// rounding mode); NaN stays a NaN.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Two fp32 -> packed pair of bf16 (lo = a, hi = b), one instruction.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    const bf16x2_hw v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Standard normal CDF Phi(u) = (1 + erf(u / sqrt 2)) / 2 and density
// phi(u) = exp(-u^2/2) / sqrt(2 pi), sharing one exponential: erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26,
// erf(z) = 1 - (a1 t + ... + a5 t^5) exp(-z^2), t = 1 / (1 + p z), z >= 0,
// absolute error <= 1.5e-7 (so |Phi error| <= 7.5e-8), on the hardware
// exp2 and reciprocal units.
__device__ __forceinline__ float normal_cdf_pdf(float u, float& pdf) {
    const float z = fabsf(u) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    const float e = __builtin_amdgcn_exp2f(-0.72134752044448170f * u * u);  // exp(-u^2/2) = 2^(-u^2 log2(e)/2)
    const float poly =
        t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f), 0.254829592f);
    const float tail = 0.5f * poly * e;  // Phi(-|u|)
    pdf = 0.39894228040143268f * e;
    return u >= 0.f ? 1.0f - tail : tail;
}

// GeLU(u) = u * Phi(u) (the erf form, not the tanh approximation).
__device__ __forceinline__ float gelu_f(float u) {
    float pdf;
    return u * normal_cdf_pdf(u, pdf);
}

// d/du GeLU(u) = Phi(u) + u * phi(u).
__device__ __forceinline__ float gelu_prime_f(float u) {
    float pdf;
    const float Phi = normal_cdf_pdf(u, pdf);
    return fmaf(u, pdf, Phi);
}

// The tanh approximation of GeLU, 0.5 u (1 + tanh(z)) with z = c (u + a u^3),
// c = sqrt(2/pi), a = 0.044715, evaluated through 1 + tanh(z) = 2 s, s = 1/(1 + e^(-2z))
// (hardware exp2 and reciprocal): GeLU = u s, with no cancellation where tanh(z)
// nears -1 (the limits come out exactly: e^(-2z) -> inf gives s = 0, -> 0 gives s = 1).
__device__ __forceinline__ float gelu_tanh_s(float u) {
    const float z = 0.7978845608028654f * fmaf(0.044715f * u, u * u, u);
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.8853900817779268f * z));  // 2 log2(e)
}

__device__ __forceinline__ float gelu_tanh_f(float u) { return u * gelu_tanh_s(u); }

// Its derivative: s + u * 2 s (1 - s) * dz/du, dz/du = c (1 + 3 a u^2).
__device__ __forceinline__ float gelu_tanh_prime_f(float u) {
    const float sg = gelu_tanh_s(u);
    const float dz = 0.7978845608028654f * fmaf(0.134145f * u, u, 1.0f);
    return fmaf(2.0f * u * sg * (1.0f - sg), dz, sg);
}

__device__ __forceinline__ float gelu_sel(float u, bool tanh_form) { return tanh_form ? gelu_tanh_f(u) : gelu_f(u); }

// GeLU(u) and, in `d`, GeLU'(u) from one evaluation of Phi and phi (erf form) or
// of s (tanh form): the values gelu_sel and gelu_prime_sel return.
__device__ __forceinline__ float gelu_and_prime(float u, bool tanh_form, float& d) {
    if (tanh_form) {
        const float sg = gelu_tanh_s(u);
        const float dz = 0.7978845608028654f * fmaf(0.134145f * u, u, 1.0f);
        d = fmaf(2.0f * u * sg * (1.0f - sg), dz, sg);
        return u * sg;
    }
    float pdf;
    const float Phi = normal_cdf_pdf(u, pdf);
    d = fmaf(u, pdf, Phi);
    return u * Phi;
}
__device__ __forceinline__ float gelu_prime_sel(float u, bool tanh_form) {
    return tanh_form ? gelu_tanh_prime_f(u) : gelu_prime_f(u);
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_hw;

// Bit-level reinterpretations between 16-byte vector types.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

// 32x32x16 bf16 MFMA.  A: lane l holds row l%32, k = 8*(l/32) .. +7;
// B: lane l holds column l%32, same k; D: lane l holds column l%32, rows
// 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 32x32x16 fp16 MFMA, same operand and result layout as the bf16 one.
__device__ __forceinline__ f32x16 mfma32x32x16_f16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

// The 16-bit storage formats: widening of the low / high half of a packed
// word, rounding of a pair to a packed word (round to nearest even), and the
// matching 32x32x16 MFMA.
template <typename T> struct Store16;
template <> struct Store16<bf16_t> {
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf2(a, b); }
    static __device__ __forceinline__ uint16_t from_f(float f) { return f2bf(f); }
    static __device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
        return mfma32x32x16(a, b, c);
    }
};
template <> struct Store16<f16_t> {
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        const f16x2_hw v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ uint16_t from_f(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
    static __device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
        return mfma32x32x16_f16(a, b, c);
    }
};

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f<f16_t>(f16_t v) { return (float)__builtin_bit_cast(_Float16, v.bits); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ f16_t from_f<f16_t>(float v) { return f16_t{__builtin_bit_cast(uint16_t, (_Float16)v)}; }

}  // namespace tp
