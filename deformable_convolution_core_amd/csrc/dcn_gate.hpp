// dcn_gate.hpp -- the centre-feature gate of the DCNv4 layer: per pixel and
// group, a sigmoid of one logit blends the sampled result y with the
// layer's projected input v (the page on the DCNv3 pure-PyTorch fallback,
// section 3, describes this sigmoid gate between the centre pixel's features
// and the sampling result).
//
//   out = y * (1 - s) + v * s,   s = 1 / (1 + exp(-z))
//
// One lane owns one (pixel, group): its Cg channels of y, v and out (and of
// the gradients), read and written in 16-byte vectors where the rows allow.
// Arithmetic is binary32.  With e = exp(-|z|) in (0, 1], s and 1 - s are
// 1/(1+e) and e/(1+e) (swapped for z < 0), so neither loses relative
// precision when the other approaches 1 and nothing overflows.
#pragma once

namespace dcn {

constexpr int kGateBlock = 256;

// VB bytes at p (VB = 16, or one element), widened to floats.
template <typename T, int VB>
__device__ __forceinline__ void gate_load(const char* p, float* f)
{
    if constexpr (VB == 16) {
        const uint4 u = *(const uint4*)p;
        const uint32_t d[4] = {u.x, u.y, u.z, u.w};
        if constexpr (Elem<T>::bytes == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(d[e]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = Elem<T>::widen(d[q] & 0xffffu);
                f[2 * q + 1] = Elem<T>::widen(d[q] >> 16);
            }
        }
    } else {
        static_assert(VB == Elem<T>::bytes, "gate vector width");
        f[0] = ld1((const T*)p);
    }
}

// (gate_weights, the s, 1 - s and s (1 - s) of a logit, is in dcn_kernels.hpp:
// the tiled forward applies the same gate in its epilogue.)

template <typename T, int VB>
__global__ __launch_bounds__(kGateBlock) void dcn_gate_forward_kernel(const char* y, const char* v, const char* z,
                                                                      char* out, uint64_t rows, uint32_t row_bytes)
{
    constexpr int EB = Elem<T>::bytes, E = VB / EB;
    const uint64_t r = (uint64_t)blockIdx.x * kGateBlock + threadIdx.x;
    if (r >= rows) return;
    const GateWeights w = gate_weights(ld1((const T*)(z + r * EB)));
    const size_t base = (size_t)r * row_bytes;
    for (uint32_t c = 0; c < row_bytes; c += VB) {
        float fy[E], fv[E], fo[E];
        gate_load<T, VB>(y + base + c, fy);
        gate_load<T, VB>(v + base + c, fv);
#pragma unroll
        for (int e = 0; e < E; ++e) fo[e] = fmaf(w.s, fv[e], w.t * fy[e]);
        store<T, VB>(out + base + c, fo);
    }
}

template <typename T, int VB>
__global__ __launch_bounds__(kGateBlock) void dcn_gate_backward_kernel(const char* y, const char* v, const char* z,
                                                                       const char* go, char* gy, char* gv, char* gz,
                                                                       uint64_t rows, uint32_t row_bytes)
{
    constexpr int EB = Elem<T>::bytes, E = VB / EB;
    const uint64_t r = (uint64_t)blockIdx.x * kGateBlock + threadIdx.x;
    if (r >= rows) return;
    const GateWeights w = gate_weights(ld1((const T*)(z + r * EB)));
    const size_t base = (size_t)r * row_bytes;
    float dot = 0.f;
    for (uint32_t c = 0; c < row_bytes; c += VB) {
        float fy[E], fv[E], fg[E], oy[E], ov[E];
        gate_load<T, VB>(y + base + c, fy);
        gate_load<T, VB>(v + base + c, fv);
        gate_load<T, VB>(go + base + c, fg);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            dot = fmaf(fg[e], fv[e] - fy[e], dot);
            oy[e] = fg[e] * w.t;
            ov[e] = fg[e] * w.s;
        }
        store<T, VB>(gy + base + c, oy);
        store<T, VB>(gv + base + c, ov);
    }
    const float d = dot * w.st;
    store<T, EB>(gz + r * EB, &d);
}

}  // namespace dcn
