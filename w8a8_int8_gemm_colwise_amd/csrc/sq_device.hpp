// sq_device.hpp -- device-side helpers shared by the library's HIP kernels.
//
// Arithmetic rules (the library is built with -ffp-contract=off): every fp32
// expression below is one IEEE operation rounded to nearest even, unless an
// explicit fused multiply-add is written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

constexpr float kFloor = 1e-7f;   // floor of every absolute maximum
constexpr float kQmax = 127.0f;   // symmetric int8 code range [-127, 127]

// Eight consecutive elements of a row, the unit of every vector load.
constexpr int kChunk = 8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load the 8 elements of chunk c of a row as fp32 (bf16 widening is exact).
template <typename T>
__device__ __forceinline__ void load_chunk(const T* row, int64_t c, float (&v)[kChunk]);

template <>
__device__ __forceinline__ void load_chunk<uint16_t>(const uint16_t* row, int64_t c,
                                                     float (&v)[kChunk]) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + c * kChunk);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}

template <>
__device__ __forceinline__ void load_chunk<float>(const float* row, int64_t c,
                                                  float (&v)[kChunk]) {
    const float4 a = *reinterpret_cast<const float4*>(row + c * kChunk);
    const float4 b = *reinterpret_cast<const float4*>(row + c * kChunk + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Raw 16-byte-granular chunk storage, so loads can be issued before use.
template <typename T> struct RawChunk;
template <> struct RawChunk<uint16_t> { uint4 u; };
template <> struct RawChunk<float> { uint4 a, b; };

template <typename T>
__device__ __forceinline__ RawChunk<T> load_raw(const T* row, int64_t c);
template <>
__device__ __forceinline__ RawChunk<uint16_t> load_raw<uint16_t>(const uint16_t* row, int64_t c) {
    return RawChunk<uint16_t>{*reinterpret_cast<const uint4*>(row + c * kChunk)};
}
template <>
__device__ __forceinline__ RawChunk<float> load_raw<float>(const float* row, int64_t c) {
    const uint4* p = reinterpret_cast<const uint4*>(row + c * kChunk);
    return RawChunk<float>{p[0], p[1]};
}

// Global-memory access through a uniform base plus a 32-bit byte offset (the
// scalar-base load form, one offset register per access; every row and
// vector here lies far below 4 GiB).  Vector types are plain ext_vector
// types: HIP's vector classes cannot be copied out of address space 1.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) char g_cchar;
typedef __attribute__((address_space(1))) char g_char;
typedef const __attribute__((address_space(1))) u32x4_t g_cu32x4;
typedef __attribute__((address_space(1))) u32x2_t g_u32x2;

__device__ __forceinline__ uint4 gload16(g_cchar* p) {
    const u32x4_t v = *(g_cu32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Eight fp32 values (32 bytes) at p.
__device__ __forceinline__ void gload8f(g_cchar* p, float (&v)[kChunk]) {
    const uint4 a = gload16(p), b = gload16(p + 16);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

__device__ __forceinline__ void gstore8(g_char* p, uint2 v) {
    *(g_u32x2*)p = u32x2_t{v.x, v.y};
}

__device__ __forceinline__ void unpack(const RawChunk<uint16_t>& r, float* v) {
    v[0] = bf16_lo(r.u.x); v[1] = bf16_hi(r.u.x);
    v[2] = bf16_lo(r.u.y); v[3] = bf16_hi(r.u.y);
    v[4] = bf16_lo(r.u.z); v[5] = bf16_hi(r.u.z);
    v[6] = bf16_lo(r.u.w); v[7] = bf16_hi(r.u.w);
}
__device__ __forceinline__ void unpack(const RawChunk<float>& r, float* v) {
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
    v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
    v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
}

// Correctly rounded reciprocal RN(1/b).  For 2^-126 <= b < 2^126 the
// hardware estimate r = v_rcp_f32(b) followed by one Newton step in fma,
// RN(r + r * RN(1 - b*r)), equals the IEEE quotient 1.0f / b: checked on gfx950
// for every float in that range against the compiler's correctly rounded
// division (the only mismatches among positive normal b lie at b >= 2^126,
// where 1/b is subnormal and the estimate flushes it).  Elsewhere (and for
// b <= 0, NaN) the IEEE division itself.  Three VALU operations and a range
// test instead of the division sequence.
__device__ __forceinline__ float rcp_rn(float b) {
    if (b >= 0x1p-126f && b < 0x1p126f) {
        const float r = __builtin_amdgcn_rcpf(b);
        return __builtin_fmaf(__builtin_fmaf(-b, r, 1.0f), r, r);
    }
    return 1.0f / b;
}

// Correctly rounded quotient RN(a / b) for b > 0 normal, given rb = RN(1/b)
// (rcp_rn or an IEEE division).  q0 = RN(a*rb) is within 1.5 ulp of a/b;
// one residual step brings it within 1 ulp; by Markstein's theorem (residual
// r = a - b*q exact, then RN(q + r*rb) with rb within half an ulp of 1/b) the
// second step returns the correctly rounded quotient.  Valid whenever the
// residuals do not underflow (|a/b| above ~2^-100) -- smaller quotients only
// ever reach rne() as 0 or an absolute maximum below the floor -- and a/b
// does not overflow.  Five VALU operations instead of the ten-instruction
// IEEE division sequence.
__device__ __forceinline__ float div_rn(float a, float b, float rb) {
    float q = a * rb;
    float r = __builtin_fmaf(-b, q, a);
    q = __builtin_fmaf(r, rb, q);
    r = __builtin_fmaf(-b, q, a);
    return __builtin_fmaf(r, rb, q);
}

// RN(a / b) as div_rn when a has at most 8 significant bits (a bf16 value):
// then q0 = RN(a*rb) is always within one ulp of a/b and the first residual
// step already returns the correctly rounded quotient.  Checked on gfx950
// against the IEEE division for every bf16 significand of a and every fp32
// significand of b, with quotients in [0.5, 2) (2^31 pairs); scaling a and b
// by powers of two does not change the rounding, and the same validity range
// as div_rn applies.  Three VALU operations.
__device__ __forceinline__ float div_rn_narrow(float a, float b, float rb) {
    const float q = a * rb;
    const float r = __builtin_fmaf(-b, q, a);
    return __builtin_fmaf(r, rb, q);
}

// x / s for an activation element of storage type T: bf16 values have 8
// significant bits, so the short sequence is exact for them.
template <typename T>
__device__ __forceinline__ float div_x(float x, float s, float rs) {
    if constexpr (sizeof(T) == 2) return div_rn_narrow(x, s, rs);
    else return div_rn(x, s, rs);
}

// Quantizer step from an absolute maximum: RN(max(FLOOR, m) / 127).
__device__ __forceinline__ float step_from_absmax(float m) {
    return fmaxf(m, kFloor) / kQmax;
}

// The step d = step_from_absmax(m) and rd = RN(1/d) together, equal to the two
// IEEE divisions.  For finite m the quotient by 127 is div_rn with the
// correctly rounded constant RN(1/127) (FLOOR/127 > 2^-31, so no residual
// underflows), and d then lies in [2^-31, 2^121), where rcp_rn's two-fma
// sequence is exact; an infinite maximum takes the divisions (fmaxf already
// maps NaN to FLOOR).  About ten VALU operations instead of two division
// sequences; m is the same in every lane that forms a row's step, so the
// branch does not diverge.
__device__ __forceinline__ void step_rcp(float m, float& d, float& rd) {
    constexpr float kRcpQmax = 1.0f / kQmax;
    const float a = fmaxf(m, kFloor);
    if (a < __builtin_inff()) {
        d = div_rn(a, kQmax, kRcpQmax);
        const float r = __builtin_amdgcn_rcpf(d);
        rd = __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
    } else {
        d = a / kQmax;
        rd = 1.0f / d;
    }
}

// rne then clamp to [-127, 127], as an int.
__device__ __forceinline__ int code_of(float q) {
    float r = __builtin_rintf(q);
    r = fminf(fmaxf(r, -kQmax), kQmax);
    return static_cast<int>(r);
}

// rne of a quotient |q| < 2^22, with the int8 code in the low byte of the
// result: q + 1.5 * 2^23 lands in [2^23, 2^24), where the fp32 spacing is 1, so
// the addition itself rounds q to the nearest integer (ties to even, the
// default rounding mode), and the low bits of the sum's bit pattern hold that
// integer in two's complement (the bit pattern of 1.5 * 2^23 ends in 22 zero
// bits).  CLAMP: the quotient is first clamped to [-127, 127], which equals
// clamping the rounded value; without it the caller guarantees |q| < 127.5.
template <bool CLAMP>
__device__ __forceinline__ uint32_t code_bits(float q) {
    if (CLAMP) q = __builtin_amdgcn_fmed3f(q, -kQmax, kQmax);
    return __float_as_uint(q + 12582912.0f);
}

// Codes of a chunk of eight values with step d (rd = RN(1/d), correctly
// rounded): q[e] = code_bits<CLAMP>(div_rn(v[e], d, rd)) for |v / d| <= 128,
// in 3.5 operations per element instead of 6.  The short form rounds the
// exact product P = v * rd to an integer in one fma, c = RN(P + 1.5 * 2^23)
// (spacing 1 there, ties to even), and keeps the residual t = RN(P - (c -
// 1.5 * 2^23)).  With Q = v / d: |P - Q| <= 2^-24 |Q| < 7.7e-6 and |RN(Q) - Q|
// <= 2^-17 / 2 (half an ulp below 128), so when |t| < 0.5 - 2^-15 the
// values P, Q and RN(Q) lie strictly between the same two half-integers: the
// integer nearest P is rne(RN(Q)), and RN(Q) is no tie.  Otherwise (about one
// chunk in 2000 of random data, and every exact tie) the lane recomputes its
// chunk with div_rn.  A NaN residual (infinite or NaN operands) does not raise
// the maximum; the sums' low bytes then match the division's (zero).
template <bool CLAMP>
__device__ __forceinline__ void chunk_codes(const float (&v)[kChunk], float d, float rd,
                                            uint32_t (&q)[kChunk]) {
    constexpr float kM = 12582912.0f;              // 1.5 * 2^23
    constexpr float kNear = 0.5f - 0x1p-15f;
    float far = 0.0f;
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
        const float c = __builtin_fmaf(v[e], rd, kM);
        const float t = __builtin_fmaf(v[e], rd, -(c - kM));
        far = fmaxf(far, fabsf(t));
        // clamping M + k to M +- 127 is clamping the rounded integer k
        q[e] = __float_as_uint(CLAMP ? __builtin_amdgcn_fmed3f(c, kM - kQmax, kM + kQmax) : c);
    }
    if (far >= kNear) {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) q[e] = code_bits<CLAMP>(div_rn(v[e], d, rd));
    }
}

// Pack the low bytes of 8 words from code_bits (byte i = element i).
__device__ __forceinline__ uint2 pack8_bits(const uint32_t (&b)[kChunk]) {
    const uint32_t p01 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
    const uint32_t p45 = __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u);
    const uint32_t p67 = __builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u);
    return make_uint2(__builtin_amdgcn_perm(p23, p01, 0x05040100u),
                      __builtin_amdgcn_perm(p67, p45, 0x05040100u));
}

// Wave-wide (64 lanes) maximum, result valid in every lane.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), d, 64)));
    return v;
}

}  // namespace sq
