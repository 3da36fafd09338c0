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
constexpr int kLinSU = 8;        // w chunks a thread has in flight while staging

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
// reads on distinct banks), then one 16 x 68-element x buffer per wave.
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
    // stage W[n0 : n0 + 64, :] in chunks of four elements, kLinSU chunks per
    // thread in flight at a time (one read latency per group, not per
    // chunk); rows past N are zero
    const int kq = K >> 2, total = kLinNB * kq;
    for (int e0 = t; e0 < total; e0 += kLinBlock * kLinSU) {
        LinFrag<T> f[kLinSU];
#pragma unroll
        for (int u = 0; u < kLinSU; ++u) {
            const int e = e0 + u * kLinBlock;
            const int r = e / kq, c = (e - r * kq) * 4;
            f[u] = (e < total && r < nb) ? lin_load<T>(W + (size_t)(n0 + r) * K + c) : lin_zero<T>();
        }
#pragma unroll
        for (int u = 0; u < kLinSU; ++u) {
            const int e = e0 + u * kLinBlock;
            if (e >= total) break;
            const int r = e / kq, c = (e - r * kq) * 4;
            if constexpr (EB == 4) *(uint4*)(wl + r * S + c) = make_uint4(f[u].d[0], f[u].d[1], f[u].d[2], f[u].d[3]);
            else *(uint2*)(wl + r * S + c) = make_uint2(f[u].d[0], f[u].d[1]);
        }
    }
    __syncthreads();

    const int ntiles = (nb + 15) >> 4;           // 16-column blocks with any valid column (stores)
    const int q = l >> 4, r16 = l & 15;
    // this lane's 16 bias values: unconditional reads at a clamped index (so
    // all 16 are in flight together), zeroed past N afterwards
    float bias[kLinNB / 16][4];
#pragma unroll
    for (int b = 0; b < kLinNB / 16; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[b][i] = 0.f;
    if (a.bias) {
        const T* bp = (const T*)a.bias;
#pragma unroll
        for (int b = 0; b < kLinNB / 16; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = n0 + 16 * b + 4 * q + i;
                bias[b][i] = ld1(bp + (n < N ? n : N - 1));
            }
#pragma unroll
        for (int b = 0; b < kLinNB / 16; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n0 + 16 * b + 4 * q + i >= N) bias[b][i] = 0.f;
    }
    const bool vec_store = (N & 3) == 0;
    const int kfull = K & ~15;
    const int nc = kfull >> 6;                   // full 64-wide chunks of k per tile
    const uint32_t stride = gridDim.x * 4u;
    // x of one 64-wide chunk of a 16-row tile is read with whole 16-byte
    // accesses, each instruction covering whole rows of the chunk
    // (contiguous in memory), into this wave's LDS buffer; the matrix
    // operands are then picked out of LDS (rows padded by four elements so a
    // 16-lane group's reads fall on distinct banks).
    constexpr int E16 = 16 / EB;                  // elements per 16-byte access
    constexpr int LPR = 64 / E16;                 // lanes per 64-element row chunk
    constexpr int RPI = 64 / LPR;                 // rows per instruction
    constexpr int NI = 16 / RPI;                  // instructions per chunk
    constexpr int XS = 64 + 4;                    // LDS row stride of the x buffer (elements)
    T* xl = wl + kLinNB * S + wave * 16 * XS;     // (half precision only)
    auto load_chunk = [&](uint32_t mtile, int chunk, uint4* raw) {
#pragma unroll
        for (int h = 0; h < NI; ++h) {
            const uint64_t row = (uint64_t)mtile * 16u + (uint32_t)(h * RPI + l / LPR);
            const T* p = X + (row < a.M ? row : a.M - 1) * (uint64_t)K + chunk * 64 + (l % LPR) * E16;
            raw[h] = *(const uint4*)p;
        }
    };
    auto put_chunk = [&](const uint4* raw) {
#pragma unroll
        for (int h = 0; h < NI; ++h) {
            T* d = xl + (h * RPI + l / LPR) * XS + (l % LPR) * E16;
            if constexpr (EB == 4) {
                *(uint4*)d = raw[h];
            } else {   // rows of 136 bytes: 8-byte aligned
                *(uint2*)d = make_uint2(raw[h].x, raw[h].y);
                *(uint2*)(d + 4) = make_uint2(raw[h].z, raw[h].w);
            }
        }
    };
    // store one finished 16-row tile: bias, one rounding, four consecutive
    // outputs per lane (element stores where N is not a multiple of 4)
    auto finish = [&](uint32_t mtile, const lin_f4* acc) {
        const uint64_t m = (uint64_t)mtile * 16u + (uint32_t)r16;
        if (m >= a.M) return;
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
    };
    // the 16-wide steps past the full chunks, then a guarded partial step
    // when K is not a multiple of 16
    auto rest = [&](uint32_t mtile, lin_f4* acc) {
        const uint64_t row = (uint64_t)mtile * 16u + (uint32_t)r16;
        const T* xrow = X + (row < a.M ? row : a.M - 1) * (uint64_t)K;
        for (int k0 = nc * 64; k0 < kfull; k0 += 16) {
            const LinFrag<T> xb = lin_load<T>(xrow + k0 + 4 * q);
#pragma unroll
            for (int b = 0; b < kLinNB / 16; ++b)
                acc[b] = lin_mfma<T>(lin_load<T>(wl + (16 * b + r16) * S + k0 + 4 * q), xb, acc[b]);
        }
        if (kfull < K) {
            const int kk = kfull + 4 * q;
            const bool in = kk < K;
            const LinFrag<T> xb = in ? lin_load<T>(xrow + kk) : lin_zero<T>();
#pragma unroll
            for (int b = 0; b < kLinNB / 16; ++b) {
                const LinFrag<T> wa = in ? lin_load<T>(wl + (16 * b + r16) * S + kk) : lin_zero<T>();
                acc[b] = lin_mfma<T>(wa, xb, acc[b]);
            }
        }
    };

    const uint32_t first = blockIdx.x * 4u + (uint32_t)wave;
    const uint32_t my_tiles = first < a.m_tiles ? (a.m_tiles - first + stride - 1) / stride : 0u;
    lin_f4 acc[kLinNB / 16];
    if (nc == 0) {
        // K < 64: no full chunk to stream
        for (uint32_t i = 0; i < my_tiles; ++i) {
            const uint32_t mtile = first + i * stride;
#pragma unroll
            for (int b = 0; b < kLinNB / 16; ++b) acc[b] = lin_f4{0.f, 0.f, 0.f, 0.f};
            rest(mtile, acc);
            finish(mtile, acc);
        }
        return;
    }
    const uint32_t nchunks = my_tiles * (uint32_t)nc;
    if constexpr (EB == 2) {
        // The full chunks of this wave's tiles form one stream: chunk s+1 is
        // read from memory into registers while chunk s multiplies out of
        // the LDS buffer.  Every branch is uniform per wave; the buffer is
        // the wave's own, and its LDS accesses complete in order, so no
        // barrier is needed.
        auto step = [&](uint32_t s_) {
            const uint32_t i = s_ / (uint32_t)nc;
            const int c = (int)(s_ - i * (uint32_t)nc);
            if (c == 0) {
#pragma unroll
                for (int b = 0; b < kLinNB / 16; ++b) acc[b] = lin_f4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const LinFrag<T> xb = lin_load<T>(xl + r16 * XS + 16 * u + 4 * q);
#pragma unroll
                for (int b = 0; b < kLinNB / 16; ++b)
                    acc[b] = lin_mfma<T>(lin_load<T>(wl + (16 * b + r16) * S + c * 64 + 16 * u + 4 * q), xb,
                                         acc[b]);
            }
            if (c == nc - 1) {
                const uint32_t mtile = first + i * stride;
                rest(mtile, acc);
                finish(mtile, acc);
            }
        };
        uint4 raw[NI];
        if (nchunks > 0) load_chunk(first, 0, raw);
        for (uint32_t s_ = 0; s_ < nchunks; ++s_) {
            put_chunk(raw);
            if (s_ + 1 < nchunks) {
                const uint32_t i = (s_ + 1) / (uint32_t)nc;
                load_chunk(first + i * stride, (int)(s_ + 1 - i * (uint32_t)nc), raw);
            }
            step(s_);
        }
    } else {
        // binary32: a lane's four consecutive x elements are already one
        // 16-byte read, so the operands come straight from memory, two chunks
        // in two register sets (one streams in while the other multiplies)
        auto direct_chunk = [&](uint32_t s_, LinFrag<T>* dst) {
            const uint32_t i = s_ / (uint32_t)nc;
            const uint64_t row = (uint64_t)(first + i * stride) * 16u + (uint32_t)r16;
            const T* p = X + (row < a.M ? row : a.M - 1) * (uint64_t)K + (s_ - i * (uint32_t)nc) * 64 + 4 * q;
#pragma unroll
            for (int u = 0; u < 4; ++u) dst[u] = lin_load<T>(p + 16 * u);
        };
        auto step = [&](uint32_t s_, const LinFrag<T>* xs) {
            const uint32_t i = s_ / (uint32_t)nc;
            const int c = (int)(s_ - i * (uint32_t)nc);
            if (c == 0) {
#pragma unroll
                for (int b = 0; b < kLinNB / 16; ++b) acc[b] = lin_f4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int b = 0; b < kLinNB / 16; ++b)
                    acc[b] = lin_mfma<T>(lin_load<T>(wl + (16 * b + r16) * S + c * 64 + 16 * u + 4 * q), xs[u],
                                         acc[b]);
            if (c == nc - 1) {
                const uint32_t mtile = first + i * stride;
                rest(mtile, acc);
                finish(mtile, acc);
            }
        };
        LinFrag<T> xa[4], xb[4];
        if (nchunks > 0) direct_chunk(0, xa);
        for (uint32_t s_ = 0; s_ < nchunks; s_ += 2) {
            if (s_ + 1 < nchunks) direct_chunk(s_ + 1, xb);
            step(s_, xa);
            if (s_ + 1 < nchunks) {
                if (s_ + 2 < nchunks) direct_chunk(s_ + 2, xa);
                step(s_ + 1, xb);
            }
        }
    }
}

}  // namespace dcn
