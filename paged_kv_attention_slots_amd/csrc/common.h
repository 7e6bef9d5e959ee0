// Device helpers shared by the msgl kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MSGL_DEV __device__ __forceinline__

namespace msgl {

typedef uint16_t bf16_t;  // bf16 in storage: raw 16-bit word

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Widen the low / high bf16 of a packed word to float (exact).
MSGL_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MSGL_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16, round to nearest even (NaN stays NaN).
MSGL_DEV uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float floatx2_t;

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
MSGL_DEV uint32_t pack_bf16x2(float lo, float hi) {
    const floatx2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// fp32 += a.bf16[0]*b.bf16[0] + a.bf16[1]*b.bf16[1]
MSGL_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

MSGL_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane movement within 16-lane rows.
template <int CTRL>
MSGL_DEV float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8-lane halves
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16-lane rows

// Sum over aligned groups of N lanes (N in {2,4,8,16,32}); every lane of a
// group receives the group's total.
template <int N>
MSGL_DEV float group_sum(float x) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group size");
    x += dpp<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    return x;
}

// Storage traits.
template <typename T>
struct Store;

template <>
struct Store<float> {
    static constexpr int kEpl = 4;  // elements per 16-byte vector
    MSGL_DEV static void widen(const uint4 &v, float (&f)[4]) {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    MSGL_DEV static uint4 narrow(const float (&f)[4]) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

template <>
struct Store<bf16_t> {
    static constexpr int kEpl = 8;
    MSGL_DEV static void widen(const uint4 &v, float (&f)[8]) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    MSGL_DEV static uint4 narrow(const float (&f)[8]) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

MSGL_DEV uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
// Streaming 16-byte load (read once; hint the caches not to keep it).
MSGL_DEV uint4 ld16_nt(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
MSGL_DEV void st16(void *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace msgl
