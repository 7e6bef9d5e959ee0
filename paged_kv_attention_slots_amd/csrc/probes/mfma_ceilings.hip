// Matrix-core ceilings for the prefill kernel's inner loop (measurement only;
// not part of libmsgl).  Each block loops over "units" of the prefill tile
// loop's shape, 32 keys x 32 query columns per wave half:
//   - S^T = K Q^T: 8 v_mfma_f32_32x32x16_bf16, A = 32 keys x 16 dims, B = Q^T
//     held in registers;
//   - O^T += V^T P^T: 8 more, A = V^T (32 dims x 16 keys), B = P^T from the
//     previous unit's scores rounded to bf16.
// Variants: operands A from registers (the matrix cores alone), or read from
// LDS with the prefill kernel's reads (16-byte K rows, transposing 8-byte V
// reads), with or without a softmax-like vector load per unit (an fma and an
// exp2 per score, bf16 packs, a rounded sum); 32 or 64 query columns per wave
// (64: two column halves share every K and V read).  LDS holds one K tile and
// one V tile of 64 rows x 256 bytes copied from the input buffer, so the
// matrix cores multiply the caller's data (random or zero: the clock, and so
// the rate, depends on it).  Thread 0 of every block records the shader clock
// cycles and the 100 MHz constant clock across its loop, so the caller can
// compute the clock the loop ran at.
// Every LDS address stays within the 32 KB tile pair: rows < 64, 16-byte chunks
// < 16 of 256-byte rows; the input buffer holds at least 32 KB.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float floatx2;

__device__ __forceinline__ floatx16 mma(const bf16x8 &a, const bf16x8 &b, const floatx16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint2 read_tr(uint32_t addr) {
    const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4 *)(uintptr_t)addr);
    return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ bf16x8 read16(uint32_t addr) {
    return *(const __attribute__((address_space(3))) bf16x8 *)(uintptr_t)addr;
}

// Row permutation of 16-byte chunks (the prefill kernel's: conflict-free
// column reads of K rows and transposing reads of V rows).
__device__ __forceinline__ int chunk_code(int r) {
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 3);
}

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const floatx2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// c + the sum of the two bf16 halves of w (a dot product with a pair of ones).
__device__ __forceinline__ float add_pair(uint32_t w, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), c,
                                           false);
}

// NC = 1: 4 waves, two blocks per CU; NC = 2: 8 waves, one block per CU (two waves per SIMD either way)
template <int NC, bool LDSRD, bool SOFTMAX>
__global__ __launch_bounds__(256 * NC, 3 - NC) void mfma_loop(const uint4 *__restrict__ src, int units, float *sink, unsigned long long *clk, int keep) {
    __shared__ __attribute__((aligned(1024))) char smem[32768];
    const int nthreads = blockDim.x;
    for (int i = threadIdx.x; i < 2048; i += nthreads) reinterpret_cast<uint4 *>(smem)[i] = src[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, jj = lane >> 5, wave = threadIdx.x >> 6;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

    bf16x8 qv[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
            qv[c][dc] = __builtin_bit_cast(bf16x8, src[((c * 8 + dc) * 64 + lane + 3 * wave) & 2047]);
    uint32_t kaddr[8], vaddr[4][2];
    {
        const int kx = chunk_code(lane & 15) ^ jj;
        const int vrow = 4 * jj + ((lane >> 2) & 3);
        const int vch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) kaddr[dc] = lds0 + (lane & 31) * 256 + (((2 * dc) ^ kx) << 4);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int par = 0; par < 2; ++par)
                vaddr[db][par] = lds0 + 16384 + vrow * 256 + (((4 * db + vch) ^ chunk_code(vrow + 8 * par)) << 4) +
                                 (lane & 1) * 8;
    }
    floatx16 acc[NC][4];
    bf16x8 pb[NC][2];
    float rsum[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[c][db] = floatx16{};
        pb[c][0] = qv[c][0];
        pb[c][1] = qv[c][1];
        rsum[c] = 0.0f;
    }
    const unsigned long long c0 = __builtin_readcyclecounter(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int u = 0; u < units; ++u) {
        const uint32_t half = (u & 1) * 32 * 256;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            uint2 av[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                if constexpr (LDSRD) {
                    av[qq] = read_tr(vaddr[db][qq & 1] + half + 8 * qq * 256);
                } else {
                    const uint4 w = __builtin_bit_cast(uint4, qv[0][(2 * db + qq) & 7]);
                    av[qq] = make_uint2(w.x, w.w);
                }
            }
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, make_uint4(av[0].x, av[0].y, av[1].x, av[1].y));
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, make_uint4(av[2].x, av[2].y, av[3].x, av[3].y));
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                acc[c][db] = mma(a0, pb[c][0], acc[c][db]);
                acc[c][db] = mma(a1, pb[c][1], acc[c][db]);
            }
        }
        floatx16 s[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) s[c] = floatx16{};
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) {
            const bf16x8 k = LDSRD ? read16(kaddr[dc] + half) : qv[0][(dc + 3) & 7];
#pragma unroll
            for (int c = 0; c < NC; ++c) s[c] = mma(k, qv[c][dc], s[c]);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            uint32_t pw[8];
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                if constexpr (SOFTMAX) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[c][e], 0.09f, -0.5f * c));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[c][e + 1], 0.09f, -0.5f * c));
                    pw[e >> 1] = pack2(p0, p1);
                    rsum[c] = add_pair(pw[e >> 1], rsum[c]);
                } else {
                    pw[e >> 1] = pack2(s[c][e], s[c][e + 1]);
                }
            }
            pb[c][0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            pb[c][1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
        }
    }
    const unsigned long long c1 = __builtin_readcyclecounter(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
    if (keep) {
        float t = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            t += rsum[c];
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) t += acc[c][db][e];
        }
        sink[blockIdx.x * nthreads + threadIdx.x] = t;
    }
}

// The matrix cores alone with v_mfma_f32_16x16x32_bf16 (8 independent
// accumulators, operands from registers, the A/B roles swapped every other
// pass): the densest issue of the bf16 units, for the power-limited ceiling.
__global__ __launch_bounds__(256, 2) void mfma16_loop(const uint4 *__restrict__ src, int units, float *sink,
                                                       unsigned long long *clk, int keep) {
    typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
    const int lane = threadIdx.x & 63;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_bit_cast(bf16x8, src[(i * 64 + lane) & 2047]);
        b[i] = __builtin_bit_cast(bf16x8, src[(1024 + i * 64 + lane) & 2047]);
    }
    floatx4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = floatx4{};
    const unsigned long long c0 = __builtin_readcyclecounter(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int u = 0; u < units; ++u) {  // 32 MFMAs of 16384 flops: the flops of one 16-MFMA 32x32x16 unit, twice
#pragma unroll
        for (int k = 0; k < 16; ++k)
            acc[k & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k & 7], b[(3 * k) & 7], acc[k & 7], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < 16; ++k)
            acc[k & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[k & 7], a[(5 * k) & 7], acc[k & 7], 0, 0, 0);
    }
    const unsigned long long c1 = __builtin_readcyclecounter(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
    if (keep) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
        sink[blockIdx.x * 256 + threadIdx.x] = t;
    }
}

}  // namespace

// Variant v: 0 = matrix cores alone (operands from registers), 1 = with the LDS
// operand reads, 2 = with LDS reads and the softmax-like vector load, 3 = the
// matrix cores alone with 16x16x32 MFMAs (32 query columns only); 32 query
// columns per wave in blocks of 4 waves (two blocks per CU), or, with wide, 64
// columns per wave in blocks of 8 waves (one block per CU).  src: at least 32 KB
// of bf16 data; sink: blocks x threads floats (written only with keep);
// clk: 2 x blocks words.  Returns a hipError_t.
extern "C" int msglp_mfma_loop(int v, int wide, const void *src, int blocks, int units, float *sink,
                               unsigned long long *clk, void *stream) {
    if (blocks < 1 || units < 1 || v < 0 || v > 3 || (v == 3 && wide)) return (int)hipErrorInvalidValue;
    const hipStream_t st = (hipStream_t)stream;
    const uint4 *s = (const uint4 *)src;
    const dim3 g(blocks);
    if (v == 3) {  // 16x16x32 MFMAs alone, 4 waves per block: 2 x 16 MFMAs of 16384 flops per unit
        hipLaunchKernelGGL(mfma16_loop, g, dim3(256), 0, st, s, units, sink, clk, 0);
    } else if (!wide) {
        const dim3 t(256);
        if (v == 0) hipLaunchKernelGGL((mfma_loop<1, false, false>), g, t, 0, st, s, units, sink, clk, 0);
        if (v == 1) hipLaunchKernelGGL((mfma_loop<1, true, false>), g, t, 0, st, s, units, sink, clk, 0);
        if (v == 2) hipLaunchKernelGGL((mfma_loop<1, true, true>), g, t, 0, st, s, units, sink, clk, 0);
    } else {
        const dim3 t(512);
        if (v == 0) hipLaunchKernelGGL((mfma_loop<2, false, false>), g, t, 0, st, s, units, sink, clk, 0);
        if (v == 1) hipLaunchKernelGGL((mfma_loop<2, true, false>), g, t, 0, st, s, units, sink, clk, 0);
        if (v == 2) hipLaunchKernelGGL((mfma_loop<2, true, true>), g, t, 0, st, s, units, sink, clk, 0);
    }
    return (int)hipGetLastError();
}
