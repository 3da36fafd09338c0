// dcn_linear.hpp -- Y = X W^T + b for the projections of the DCNv4 layer
// around the sampling core: X (M, K) row-major with M in the hundreds of
// thousands, W (N, K) with K and N a few dozen to a few hundred, Y (M, N).
// At these shapes the product is bound by streaming X and Y through HBM
// (2MNK flops against (MK + MN) elements), so the kernel reads X once, keeps
// a block of W rows in LDS and lets the matrix cores do the arithmetic.
//
// Each wave computes 16-row tiles of Y as 16 x 16 blocks of Y^T with
// v_mfma_f32_16x16x16 (f16 / bf16) or v_mfma_f32_16x16x4 (f32):
//   A = W block   (16 n x 16 k): lane l holds W[n0 + l%16][k0 + 4(l/16) + i]
//   B = X^T block (16 k x 16 m): lane l holds X[m0 + l%16][k0 + 4(l/16) + i]
//   D = Y^T block (16 n x 16 m): lane l holds Y[m0 + l%16][n0 + 4(l/16) + i]
// for i = 0..3, so every operand is four consecutive elements of a row (one
// 8- or 16-byte read) and every lane writes four consecutive outputs.  The
// f32 form issues four 16x16x4 products per 16-wide step, one per element i
// (each covers k = 4q + i, q = 0..3): the same sum in another order.
// Products of half-precision operands are exact in binary32; accumulation
// and the bias add are binary32, the result is rounded once.
#pragma once

namespace dcn {

constexpr int kLinBlock = 256;   // 4 waves
constexpr int kLinNB = 64;       // columns of Y per block (W rows staged in LDS)

typedef float lin_f4 __attribute__((ext_vector_type(4)));
typedef _Float16 lin_h4 __attribute__((ext_vector_type(4)));
typedef short lin_s4 __attribute__((ext_vector_type(4)));

// four consecutive elements as MFMA operand bits (two dwords for half types,
// four for f32)
template <typename T> struct LinFrag { uint32_t d[Elem<T>::bytes == 4 ? 4 : 2]; };

template <typename T>
__device__ __forceinline__ LinFrag<T> lin_load(const T* p)
{
    LinFrag<T> f;
    if constexpr (Elem<T>::bytes == 4) {
        const uint4 v = *(const uint4*)p;
        f.d[0] = v.x; f.d[1] = v.y; f.d[2] = v.z; f.d[3] = v.w;
    } else {
        const uint2 v = *(const uint2*)p;
        f.d[0] = v.x; f.d[1] = v.y;
    }
    return f;
}

template <typename T>
__device__ __forceinline__ LinFrag<T> lin_zero()
{
    LinFrag<T> f;
#pragma unroll
    for (int i = 0; i < (Elem<T>::bytes == 4 ? 4 : 2); ++i) f.d[i] = 0u;
    return f;
}

// acc += A B for one 16-wide step of k
template <typename T>
__device__ __forceinline__ lin_f4 lin_mfma(const LinFrag<T>& a, const LinFrag<T>& b, lin_f4 acc)
{
    if constexpr (Elem<T>::bytes == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.d[i]), __uint_as_float(b.d[i]), acc, 0, 0, 0);
        return acc;
    } else if constexpr (std::is_same<T, _Float16>::value) {
        const lin_h4 av = __builtin_bit_cast(lin_h4, make_uint2(a.d[0], a.d[1]));
        const lin_h4 bv = __builtin_bit_cast(lin_h4, make_uint2(b.d[0], b.d[1]));
        return __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, acc, 0, 0, 0);
    } else {
        const lin_s4 av = __builtin_bit_cast(lin_s4, make_uint2(a.d[0], a.d[1]));
        const lin_s4 bv = __builtin_bit_cast(lin_s4, make_uint2(b.d[0], b.d[1]));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
    }
}

struct LinArgs {
    const void* x;
    const void* w;
    const void* bias;   // may be null
    void* y;
    uint64_t M;
    int N, K;
    uint32_t m_tiles;   // ceil(M / 16)
};

// grid: (blocks over 16-row tiles, ceil(N / 64)); K % 4 == 0.  LDS: 64 W rows
// at a stride of K + 4 elements (the pad puts the 16 rows one 16-lane group
// reads on distinct banks).
template <typename T>
__global__ __launch_bounds__(kLinBlock) void dcn_linear_kernel(LinArgs a)
{
    constexpr int EB = Elem<T>::bytes;
    extern __shared__ uint4 lin_lds[];
    T* wl = (T*)lin_lds;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int K = a.K, N = a.N, S = K + 4;
    const int n0 = (int)blockIdx.y * kLinNB;
    const int nb = N - n0 < kLinNB ? N - n0 : kLinNB;
    const T* W = (const T*)a.w;
    const T* X = (const T*)a.x;
    // stage W[n0 : n0 + 64, :] in chunks of four elements; rows past N are zero
    const int kq = K >> 2;
    for (int e = t; e < kLinNB * kq; e += kLinBlock) {
        const int r = e / kq, c = (e - r * kq) * 4;
        const LinFrag<T> f = r < nb ? lin_load<T>(W + (size_t)(n0 + r) * K + c) : lin_zero<T>();
        if constexpr (EB == 4) *(uint4*)(wl + r * S + c) = make_uint4(f.d[0], f.d[1], f.d[2], f.d[3]);
        else *(uint2*)(wl + r * S + c) = make_uint2(f.d[0], f.d[1]);
    }
    __syncthreads();

    const int ntiles = (nb + 15) >> 4;           // 16-column blocks with any valid column
    const int q = l >> 4, r16 = l & 15;
    float bias[kLinNB / 16][4];
#pragma unroll
    for (int b = 0; b < kLinNB / 16; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + 16 * b + 4 * q + i;
            bias[b][i] = (a.bias && n < N) ? ld1((const T*)a.bias + n) : 0.f;
        }
    const bool vec_store = (N & 3) == 0;
    for (uint32_t mt = blockIdx.x * 4u + (uint32_t)wave; mt < a.m_tiles; mt += gridDim.x * 4u) {
        const uint64_t m = (uint64_t)mt * 16u + (uint32_t)r16;
        const uint64_t mr = m < a.M ? m : a.M - 1;   // rows past M read the last row and store nothing
        const T* xrow = X + mr * (uint64_t)K;
        lin_f4 acc[kLinNB / 16];
#pragma unroll
        for (int b = 0; b < kLinNB / 16; ++b) acc[b] = lin_f4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < K; k0 += 16) {
            const int kk = k0 + 4 * q;
            const LinFrag<T> xb = kk < K ? lin_load<T>(xrow + kk) : lin_zero<T>();
#pragma unroll
            for (int b = 0; b < kLinNB / 16; ++b) {
                if (b < ntiles) {
                    const T* wp = wl + (16 * b + r16) * S + kk;
                    const LinFrag<T> wa = kk < K ? lin_load<T>(wp) : lin_zero<T>();
                    acc[b] = lin_mfma<T>(wa, xb, acc[b]);
                }
            }
        }
        if (m < a.M) {
            T* yrow = (T*)a.y + m * (uint64_t)N;
#pragma unroll
            for (int b = 0; b < kLinNB / 16; ++b) {
                if (b >= ntiles) continue;
                const int n = n0 + 16 * b + 4 * q;
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = acc[b][i] + bias[b][i];
                if (vec_store && n + 3 < N) {
                    store<T, 4 * EB>(yrow + n, v);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n + i < N) store<T, EB>(yrow + n + i, &v[i]);
                }
            }
        }
    }
}

}  // namespace dcn
