// dcn_wgrad.hpp -- weight and bias gradients of the DCNv4 layer's projections:
//   dW[o][i] = sum_m g[m][o] * x[m][i],   db[o] = sum_m g[m][o]
// with g (M, O) the gradient of a projection's output, x (M, I) its input,
// M in the hundreds of thousands and O, I a few dozen to a few hundred.  The
// reduction runs over the long dimension, so the rows are split into chunks:
// each block reduces one chunk of rows for one 128 x 64 block of dW on the
// matrix cores and writes a binary32 partial; a second kernel adds the
// partials of all chunks in a fixed order (the result does not depend on
// scheduling).
//
// The MFMA operand layout is the one of dcn_linear.hpp (lin_mfma): for a
// 16-row step of m, A = g^T (16 o x 16 m) and B = x (16 m x 16 i), lane l
// holding A[o0 + l%16][4(l/16) + e] and B[4(l/16) + e][i0 + l%16], e = 0..3,
// and D = dW block with lane l holding dW[o0 + 4(l/16) + e][i0 + l%16].  A
// lane's four operand elements lie in four rows, so a chunk of 64 rows of g
// and x is first staged in LDS with wide row reads and the operands are
// picked out of it.  The bias gradient is one more 16-column block of B whose
// first column is all ones.
#pragma once

namespace dcn {

constexpr int kWgBlock = 256;          // 4 waves
constexpr int kWgRows = 64;            // rows of g and x per staged chunk
constexpr int kWgOB = 128;             // dW rows per block (8 tiles: wave w takes tiles w and w + 4)
constexpr int kWgIB = 64;              // dW columns per block (4 tiles)
constexpr int kWgGS = kWgOB + 4;       // LDS row strides (elements): with these pads the four
constexpr int kWgXS = kWgIB + 4;       // rows one operand read spans fall on distinct banks

struct WgArgs {
    const void* g;
    const void* x;
    float* part;             // (nchunks, part_rows, part_ld) binary32 partials
    uint64_t M;
    int O, I;
    uint32_t rows_per_chunk; // a multiple of kWgRows
    int part_rows;           // ceil(O / 128) * 128
    int part_ld;             // ceil(I / 64) * 64 + 16; the last 16 columns hold the bias block
    int bias;                // nonzero: form the bias block (blocks with blockIdx.z == 0)
};

// Stage rows [m0, m0 + 64) x columns [c0, c0 + nc) of a row-major (M, ld)
// matrix into LDS at a row stride of `stride` elements, one read after
// another; rows at or past m_end are zeros.  vb: bytes per read (16 or 4,
// dividing the row segment and its start, or the element size).
template <typename T>
__device__ __forceinline__ void wg_stage(T* dst, int stride, const T* src, uint64_t ld, uint64_t m0, uint64_t m_end,
                                         int c0, int nc, int vb, int t)
{
    constexpr int EB = Elem<T>::bytes;
    const int per = vb / EB;                  // elements per read
    const int rv = nc / per;                  // reads per row
    for (int e = t; e < kWgRows * rv; e += kWgBlock) {
        const int r = e / rv, c = (e - r * rv) * per;
        const uint64_t m = m0 + (uint64_t)r;
        const T* s = src + m * ld + (uint64_t)(c0 + c);
        T* d = dst + r * stride + c;
        const bool in = m < m_end;
        if (vb == 16) {
            const uint4 v = in ? *(const uint4*)s : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (EB == 4) {
                *(uint4*)d = v;
            } else {   // LDS rows of half types are 8-byte aligned
                *(uint2*)d = make_uint2(v.x, v.y);
                *(uint2*)(d + 4) = make_uint2(v.z, v.w);
            }
        } else if (vb == 4) {
            *(uint32_t*)d = in ? *(const uint32_t*)s : 0u;
        } else {
            *d = in ? *s : (T)0.0f;
        }
    }
}

// One thread's share of a 64-row chunk of a matrix with at most CAP columns
// per block, read VB bytes at a time (VB = 16, 8 or 4, dividing the row
// segment and its start): all reads are issued together, and the chunk after
// the one being multiplied is in flight during the products.
template <typename T, int CAP, int VB>
struct WgPiece {
    static constexpr int N = kWgRows * CAP * Elem<T>::bytes / VB / kWgBlock;   // reads per thread at most
    uint32_t v[N][VB / 4];
};

// Reads go through a buffer resource over rows [m0, m_end) of the matrix, so
// rows past the end read as zeros, with 32-bit offsets (the host keeps 64
// rows under 2^31 bytes).
template <typename T, int CAP, int VB>
__device__ __forceinline__ void wg_fetch(WgPiece<T, CAP, VB>& pc, const T* src, uint64_t ld, uint64_t m0,
                                         uint64_t m_end, int c0, int nc, int t)
{
    constexpr int EB = Elem<T>::bytes, PER = VB / EB;
    const int rv = nc / PER;                       // reads per row
    const uint64_t left = (m_end - m0) * ld * EB;
    // (at most kOOB bytes, so kOOB is always out of range)
    const __amdgpu_buffer_rsrc_t r = image_rsrc(src + m0 * ld, left < kOOB ? (uint32_t)left : kOOB);
#pragma unroll
    for (int u = 0; u < WgPiece<T, CAP, VB>::N; ++u) {
        const int e = t + u * kWgBlock;
        const int row = e / rv, c = (e - row * rv) * PER;
        const uint32_t off = e < kWgRows * rv ? ((uint32_t)row * (uint32_t)ld + (uint32_t)(c0 + c)) * EB : kOOB;
        if constexpr (VB == 16) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
            pc.v[u][0] = v[0]; pc.v[u][1] = v[1]; pc.v[u][2] = v[2]; pc.v[u][3] = v[3];
        } else if constexpr (VB == 8) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            pc.v[u][0] = v[0]; pc.v[u][1] = v[1];
        } else {
            pc.v[u][0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        }
    }
}

template <typename T, int CAP, int VB>
__device__ __forceinline__ void wg_put(const WgPiece<T, CAP, VB>& pc, T* dst, int stride, int nc, int t)
{
    constexpr int EB = Elem<T>::bytes, PER = VB / EB;
    const int rv = nc / PER;
#pragma unroll
    for (int u = 0; u < WgPiece<T, CAP, VB>::N; ++u) {
        const int e = t + u * kWgBlock;
        if (e >= kWgRows * rv) break;
        const int r = e / rv, c = (e - r * rv) * PER;
        T* d = dst + r * stride + c;
        if constexpr (VB == 16 && EB == 4) {
            *(uint4*)d = make_uint4(pc.v[u][0], pc.v[u][1], pc.v[u][2], pc.v[u][3]);
        } else if constexpr (VB == 16) {   // LDS rows of half types are 8-byte aligned
            *(uint2*)d = make_uint2(pc.v[u][0], pc.v[u][1]);
            *(uint2*)(d + 4) = make_uint2(pc.v[u][2], pc.v[u][3]);
        } else if constexpr (VB == 8) {
            *(uint2*)d = make_uint2(pc.v[u][0], pc.v[u][1]);
        } else {
            *(uint32_t*)d = pc.v[u][0];
        }
    }
}

// the four operand elements of rows k + 4(l/16) + e, column col, of a staged
// chunk
template <typename T>
__device__ __forceinline__ LinFrag<T> wg_operand(const T* lds, int stride, int k, int col)
{
    LinFrag<T> f;
    if constexpr (Elem<T>::bytes == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f.d[e] = __float_as_uint(lds[(k + e) * stride + col]);
    } else {
        const uint16_t* p = (const uint16_t*)lds;
        f.d[0] = (uint32_t)p[k * stride + col] | ((uint32_t)p[(k + 1) * stride + col] << 16);
        f.d[1] = (uint32_t)p[(k + 2) * stride + col] | ((uint32_t)p[(k + 3) * stride + col] << 16);
    }
    return f;
}

// B block of the bias gradient: column 0 all ones, the rest zeros
template <typename T>
__device__ __forceinline__ LinFrag<T> wg_ones(bool first_column)
{
    LinFrag<T> f;
    if constexpr (Elem<T>::bytes == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f.d[e] = first_column ? 0x3f800000u : 0u;
    } else {
        const uint32_t one = std::is_same<T, _Float16>::value ? 0x3c00u : 0x3f80u;
        f.d[0] = f.d[1] = first_column ? (one | (one << 16)) : 0u;
    }
    return f;
}

// grid: (nchunks, ceil(O / 128), ceil(I / 64)).  VG, VX: bytes per staging
// read of g and of x rows (16, 8 or 4); both 0 for element reads (rows whose
// length or start allows no wider read).
template <typename T, int VG, int VX>
__global__ __launch_bounds__(kWgBlock) void dcn_wgrad_kernel(WgArgs a)
{
    constexpr int VB = VG;   // 0: the element path
    __shared__ T gl[kWgRows * kWgGS];
    __shared__ T xl[kWgRows * kWgXS];
    const int t = threadIdx.x, l = t & 63, w = t >> 6, q = l >> 4, r16 = l & 15;
    const int o0 = (int)blockIdx.y * kWgOB, i0 = (int)blockIdx.z * kWgIB;
    const int ob = a.O - o0 < kWgOB ? a.O - o0 : kWgOB;
    const int ib = a.I - i0 < kWgIB ? a.I - i0 : kWgIB;
    const uint64_t m_begin = (uint64_t)blockIdx.x * a.rows_per_chunk;
    const uint64_t m_end = m_begin + a.rows_per_chunk < a.M ? m_begin + a.rows_per_chunk : a.M;
    const bool bias = a.bias && blockIdx.z == 0;
    // this wave's dW row tiles (w and w + 4) and the column tiles with any
    // valid column; all wave-uniform
    const bool ot_ok[2] = {16 * w < ob, 16 * (w + 4) < ob};
    const int nit = (ib + 15) >> 4;
    lin_f4 acc[2][5];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 5; ++u) acc[j][u] = lin_f4{0.f, 0.f, 0.f, 0.f};
    const LinFrag<T> ones = wg_ones<T>(r16 == 0);

    WgPiece<T, kWgOB, VG == 0 ? 4 : VG> gp;       // (unused on the element path)
    WgPiece<T, kWgIB, VX == 0 ? 4 : VX> xp;
    if constexpr (VB != 0) {
        wg_fetch(gp, (const T*)a.g, (uint64_t)a.O, m_begin, m_end, o0, ob, t);
        wg_fetch(xp, (const T*)a.x, (uint64_t)a.I, m_begin, m_end, i0, ib, t);
    }
    for (uint64_t m0 = m_begin; m0 < m_end; m0 += kWgRows) {
        __syncthreads();   // the previous chunk's operand reads are done
        if constexpr (VB != 0) {
            wg_put(gp, gl, kWgGS, ob, t);
            wg_put(xp, xl, kWgXS, ib, t);
        } else {
            wg_stage<T>(gl, kWgGS, (const T*)a.g, (uint64_t)a.O, m0, m_end, o0, ob, Elem<T>::bytes, t);
            wg_stage<T>(xl, kWgXS, (const T*)a.x, (uint64_t)a.I, m0, m_end, i0, ib, Elem<T>::bytes, t);
        }
        __syncthreads();
        if constexpr (VB != 0) {
            if (m0 + kWgRows < m_end) {   // the next chunk, in flight during the products
                wg_fetch(gp, (const T*)a.g, (uint64_t)a.O, m0 + kWgRows, m_end, o0, ob, t);
                wg_fetch(xp, (const T*)a.x, (uint64_t)a.I, m0 + kWgRows, m_end, i0, ib, t);
            }
        }
#pragma unroll
        for (int k = 0; k < kWgRows; k += 16) {
            LinFrag<T> xb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (u < nit) xb[u] = wg_operand<T>(xl, kWgXS, k + 4 * q, 16 * u + r16);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (!ot_ok[j]) continue;
                const LinFrag<T> ga = wg_operand<T>(gl, kWgGS, k + 4 * q, 16 * (w + 4 * j) + r16);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (u < nit) acc[j][u] = lin_mfma<T>(ga, xb[u], acc[j][u]);
                if (bias) acc[j][4] = lin_mfma<T>(ga, ones, acc[j][4]);
            }
        }
    }

    // partial of this chunk: rows o0 + 16 tile + 4(l/16) + e, columns of the
    // lane; every row and column of a tile that has a valid one is written
    // (the reduction reads only valid ones)
    float* part = a.part + (uint64_t)blockIdx.x * (uint64_t)a.part_rows * (uint64_t)a.part_ld;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (!ot_ok[j]) continue;
        const int orow = o0 + 16 * (w + 4 * j) + 4 * q;
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            if (u < 4 ? u >= nit : !bias) continue;
            const int col = (u < 4 ? i0 + 16 * u : a.part_ld - 16) + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) part[(uint64_t)(orow + e) * (uint64_t)a.part_ld + (uint64_t)col] = acc[j][u][e];
        }
    }
}

constexpr int kWgRedCols = 8;      // 4-column groups per reduction block
constexpr int kWgRedGroups = 32;   // chunk groups per column group (kWgRedCols * kWgRedGroups threads)

// dw[o][i] = sum over chunks c of part[c][o][i], c in a fixed order: group
// k sums chunks k, k + 32, k + 64, ..., then the 32 group sums are added in
// order; db[o] likewise from the bias column.  The binary32 sums are stored
// rounded once to OutT.  A thread reads four consecutive partials of a row
// (16 bytes) per chunk, eight threads a 128-byte row segment; the padded
// columns are read and dropped.
template <typename OutT>
__global__ __launch_bounds__(kWgRedCols * kWgRedGroups) void dcn_wgrad_reduce(const float* part, OutT* dw, OutT* db,
                                                                              int O, int I, int part_rows,
                                                                              int part_ld, uint32_t nchunks)
{
    __shared__ float4 s[kWgRedGroups][kWgRedCols];
    const int j = threadIdx.x % kWgRedCols, grp = threadIdx.x / kWgRedCols;
    const int q4 = part_ld / 4;                                  // 4-column groups per row
    const int64_t f = (int64_t)blockIdx.x * kWgRedCols + j;      // 4-column group over rows o < O
    const bool valid = f < (int64_t)O * q4;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
        const uint64_t step = (uint64_t)part_rows * (uint64_t)part_ld / 4u;
        const float4* p = (const float4*)part + (uint64_t)f;   // row f / q4, columns 4 (f % q4) + 0..3
        uint32_t c = (uint32_t)grp;
        for (; c + 15u * kWgRedGroups < nchunks; c += 16u * kWgRedGroups) {
            float4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = p[(uint64_t)(c + (uint32_t)u * kWgRedGroups) * step];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w;
            }
        }
        for (; c < nchunks; c += kWgRedGroups) {
            const float4 v = p[(uint64_t)c * step];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
    }
    s[grp][j] = sum;
    __syncthreads();
    if (grp == 0 && valid) {
        float4 r = s[0][j];
#pragma unroll
        for (int k = 1; k < kWgRedGroups; ++k) {
            r.x += s[k][j].x; r.y += s[k][j].y; r.z += s[k][j].z; r.w += s[k][j].w;
        }
        const int o = (int)(f / q4), c0 = (int)(f % q4) * 4;
        const float rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = c0 + e;
            if (col < I) dw[(int64_t)o * I + col] = (OutT)rv[e];
            else if (db && col == part_ld - 16) db[o] = (OutT)rv[e];
        }
    }
}

// Zeros of dw and db for a call over no rows, in any output type.
template <typename OutT>
__global__ __launch_bounds__(256) void dcn_wgrad_zero(OutT* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = (OutT)0.f;
}

}  // namespace dcn
