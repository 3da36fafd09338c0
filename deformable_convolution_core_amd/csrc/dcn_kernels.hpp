// dcn_kernels.hpp -- gfx950 kernels of the deformable sampling core.
//
// Pages cited (title, site):
//   [FB]  "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读"
//         (the DCNv3 pure-PyTorch fallback read line by line), trdm.cn
//   [FII] FlashInternImage image-classification guide, m.nxbn.cn: section 2.2
//         (one fused kernel instead of several memory-bound ones; no sampled
//         intermediate written to global memory)
//   [V4]  "DCNv4高效实践指南：掌握可变形卷积的3倍速度提升技术", seekfood.cn:
//         core-architecture section (no softmax; fewer redundant memory ops)
//
// One lane owns CPL contiguous channels of one (pixel, group).  The lanes of
// a wave cover consecutive channel chunks of consecutive pixels of one image,
// so each bilinear corner read is a contiguous NHWC row segment and the
// output store of a wave is one contiguous span.  The P offsets and mask
// values of a (pixel, group) are read once per lane (the L = Cg/CPL lanes of
// a group read the same bytes, which L1 serves).  Nothing is staged through
// global memory: coordinates, weights, the optional softmax and the
// accumulation stay in registers ([FII] section 2.2).
//
// Gathers go through a buffer resource spanning exactly one image.  Every
// corner that lies off the map gets an out-of-range offset, for which the
// hardware returns zeros, so no lane reads outside the image it samples and
// off-map pixels never contaminate a sum (even if a neighbouring row holds
// a NaN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dcn {

constexpr int kBlock = 256;
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past any image (images are < 2^31 bytes)

// ---------------------------------------------------------------------------
// Division by a runtime-invariant divisor with a precomputed multiplier
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): for 1 <= d < 2^31 and x < 2^31,
// q = (umulhi(x, m) + x) >> s with s = ceil(log2 d), m = ceil(2^(32+s)/d) - 2^32.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    f.s = 0;
    while ((1ull << f.s) < d) ++f.s;
    f.m = (uint32_t)((((1ull << 32) * ((1ull << f.s) - d)) / d) + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f)
{
    return (__umulhi(x, f.m) + x) >> f.s;
}

// ---------------------------------------------------------------------------
// Element types: widened exactly to float, rounded once (nearest even) back.
template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int bytes = 4;
    __device__ static float widen(uint32_t u) { return __uint_as_float(u); }
    __device__ static uint32_t narrow(float f) { return __float_as_uint(f); }
};
template <> struct Elem<_Float16> {
    static constexpr int bytes = 2;
    __device__ static float widen(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)u); }
    __device__ static uint32_t narrow(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
};
template <> struct Elem<__bf16> {
    static constexpr int bytes = 2;
    __device__ static float widen(uint32_t u) { return __uint_as_float(u << 16); }
    __device__ static uint32_t narrow(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
};

template <typename T>
__device__ __forceinline__ float ld1(const T* p)
{
    if constexpr (sizeof(T) == 4) return *(const float*)p;
    else return Elem<T>::widen(*(const uint16_t*)p);
}

// Two consecutive elements (an offset pair).  A half-precision pair is read
// as two 16-bit loads: in the packed offset+mask record (3P elements per
// record) an odd P puts every other record on a 2-byte boundary.
template <typename T>
__device__ __forceinline__ float2 ld2(const T* p)
{
    if constexpr (sizeof(T) == 4) return *(const float2*)p;
    else {
        const uint16_t* h = (const uint16_t*)p;
        return make_float2(Elem<T>::widen(h[0]), Elem<T>::widen(h[1]));
    }
}

// Store an offset pair (the gradient of (dx, dy)); same alignment rule as ld2.
template <typename T>
__device__ __forceinline__ void store_pair(T* p, float x, float y)
{
    if constexpr (sizeof(T) == 4) {
        *(float2*)p = make_float2(x, y);
    } else {
        uint16_t* h = (uint16_t*)p;
        h[0] = (uint16_t)Elem<T>::narrow(x);
        h[1] = (uint16_t)Elem<T>::narrow(y);
    }
}

// LB bytes (LB in {2,4,8,16}, >= sizeof(T)) from a buffer resource, widened
// to LB/sizeof(T) floats.
template <typename T, int LB>
__device__ __forceinline__ void gather(__amdgpu_buffer_rsrc_t r, uint32_t off, float* f)
{
    constexpr int E = LB / Elem<T>::bytes;
    uint32_t d[LB >= 4 ? LB / 4 : 1];
    if constexpr (LB == 16) {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    } else if constexpr (LB == 8) {
        auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        d[0] = v[0]; d[1] = v[1];
    } else if constexpr (LB == 4) {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else {
        static_assert(LB == 2 && Elem<T>::bytes == 2, "load width");
        d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
    if constexpr (Elem<T>::bytes == 4) {
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = __uint_as_float(d[e]);
    } else if constexpr (LB == 2) {
        f[0] = Elem<T>::widen(d[0]);
    } else {
#pragma unroll
        for (int q = 0; q < LB / 4; ++q) {
            f[2 * q] = Elem<T>::widen(d[q] & 0xffffu);
            f[2 * q + 1] = Elem<T>::widen(d[q] >> 16);
        }
    }
}

// Store LB bytes built from LB/sizeof(T) floats (pointer LB-aligned).
template <typename T, int LB>
__device__ __forceinline__ void store(void* p, const float* f)
{
    if constexpr (LB == 2) {
        *(uint16_t*)p = (uint16_t)Elem<T>::narrow(f[0]);
    } else {
        struct alignas(LB) V { uint32_t d[LB / 4]; } v;
#pragma unroll
        for (int q = 0; q < LB / 4; ++q) {
            if constexpr (Elem<T>::bytes == 4) v.d[q] = __float_as_uint(f[q]);
            else v.d[q] = Elem<T>::narrow(f[2 * q]) | (Elem<T>::narrow(f[2 * q + 1]) << 16);
        }
        *(V*)p = v;
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t image_rsrc(const void* base, uint32_t bytes)
{
    // dword3 0x00020000: raw (unswizzled) buffer, 32-bit data format, gfx9 family
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Buffer resource over one image of offset or mask records, based on the
// dword boundary at or below the image start; lead (0 or 2) is the byte
// distance from that boundary to the image.  Half-precision records can start
// on a 2-byte boundary (a mask record of odd P, a packed record of odd P, an
// image after an odd number of them), and load_record's realignment needs
// byte offsets that are true to the address's alignment.  Reading back to the
// boundary stays inside the word that holds the image's first byte.
struct RecordRsrc {
    __amdgpu_buffer_rsrc_t r;
    uint32_t lead;
};

__device__ __forceinline__ RecordRsrc record_rsrc(const void* img, uint32_t bytes)
{
    // the range ends on a dword boundary too: a dword holding the image's
    // last bytes is read whole
    const uint32_t lead = (uint32_t)(uintptr_t)img & 3u;
    return RecordRsrc{image_rsrc((const char*)img - lead, (bytes + lead + 3u) & ~3u), lead};
}

// The hardware hands workgroup b to XCD (b mod 8).  Renumber so each XCD gets
// one contiguous range of logical tiles: neighbouring tiles, which sample
// overlapping input rows, then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nb)
{
    const uint32_t xcd = b & 7u, k = b >> 3, q = nb >> 3, r = nb & 7u;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

struct Geometry {
    int H, W, C, groups, Ho, Wo, K, P, stride, pad, dil, c0;
    int rc;                       // 1: the centre tap is left out (P = K*K - 1)
    int off_stride, mask_stride;  // elements per (pixel, group) record of offset / mask
    float alpha;
    int softmax;
    uint32_t in_image_bytes;      // H*W*C*b
    uint32_t in_row_bytes;        // C*b     (one pixel)
    uint32_t in_line_bytes;       // W*C*b   (one image row)
    uint32_t lanes_per_image;     // Ho*Wo*C/CPL
    uint32_t blocks_per_image;
    FastDiv chunks;               // C/CPL channel chunks per pixel
    FastDiv lanes_per_group;      // L = Cg/CPL
    FastDiv wo_div;               // Wo
};

// Index among the P points of tap (i, j) (p = i*K + j, with the centre
// left out under remove_center), or -1 for the left-out tap.
__device__ __forceinline__ int point_of(const Geometry& G, int i, int j)
{
    const int p = i * G.K + j, centre = (G.K * G.K - 1) >> 1;
    if (!G.rc) return p;
    return p == centre ? -1 : p - (p > centre ? 1 : 0);
}

struct FwdArgs {
    const void* input;
    const void* offset;
    const void* mask;
    void* output;
    Geometry geo;
    const void* gate;        // centre-feature gate logits (N, Ho, Wo, G), or null
    void* core_out;          // with a gate: the sampled result before the gate, or null
};

// The centre-feature gate of the DCNv4 layer: s = 1 / (1 + exp(-z)) and 1 - s
// from e = exp(-|z|) in (0, 1] as 1/(1+e) and e/(1+e) (swapped for z < 0), so
// neither loses relative precision when the other approaches 1 and nothing
// overflows; st = s (1 - s).  A NaN logit makes all three NaN.
struct GateWeights {
    float s, t, st;
};

__device__ __forceinline__ GateWeights gate_weights(float z)
{
    const float e = expf(-fabsf(z));
    const float inv = 1.0f / (1.0f + e);
    const float big = inv, small = e * inv;          // the larger and the smaller of s, 1 - s
    GateWeights w;
    w.s = z >= 0.f ? big : small;
    w.t = z >= 0.f ? small : big;
    w.st = small * inv;
    return w;
}

struct BwdArgs {
    const void* input;
    const void* offset;
    const void* mask;
    const void* grad_out;
    void* grad_input;             // all three in the call's dtype
    void* grad_offset;
    void* grad_mask;
    int near_m;                   // >= 0: corners within this many pixels of the sampling
                                  // base were added by the owner kernel; -1: none were
    Geometry geo;
};

// The (image, pixel, group, channel chunk) a lane owns.
struct LaneWork {
    uint32_t n, pix, ho, wo, g, cc;
    bool active;
};

__device__ __forceinline__ LaneWork lane_work(const Geometry& G)
{
    LaneWork w;
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    w.n = b / G.blocks_per_image;                         // wave-uniform
    const uint32_t t = (b - w.n * G.blocks_per_image) * kBlock + threadIdx.x;
    w.active = t < G.lanes_per_image;
    w.pix = fdiv(t, G.chunks);
    w.cc = t - w.pix * G.chunks.d;
    w.g = fdiv(w.cc, G.lanes_per_group);
    w.ho = fdiv(w.pix, G.wo_div);
    w.wo = w.pix - w.ho * G.Wo;
    return w;
}

// One sampling point: binary32 coordinates in the documented order, floor,
// fractions, corner validity and the four gather offsets (out of range for
// off-map corners).  Corners are 00, 01, 10, 11 = (y0,x0), (y0,x0+1),
// (y0+1,x0), (y0+1,x0+1).
struct Sample {
    float lx, ly;
    int x0, y0;                   // floor of the (parked) coordinates
    bool inmap;
    bool v[4];
    uint32_t off[4];
};

__device__ __forceinline__ Sample make_sample(const Geometry& G, float bx, float by, int i, int j,
                                              float dx, float dy, uint32_t chan_bytes)
{
    Sample s;
    float x = fmaf(G.alpha, dx, fmaf(G.alpha, (float)(i * G.dil - G.c0), bx));
    float y = fmaf(G.alpha, dy, fmaf(G.alpha, (float)(j * G.dil - G.c0), by));
    s.inmap = x > -1.0f && x < (float)G.W && y > -1.0f && y < (float)G.H;
    x = s.inmap ? x : -2.0f;          // off the map or NaN: park where no corner is valid
    y = s.inmap ? y : -2.0f;
    const float fx = floorf(x), fy = floorf(y);
    s.lx = x - fx;
    s.ly = y - fy;
    const int x0 = (int)fx, y0 = (int)fy;
    s.x0 = x0;
    s.y0 = y0;
    const bool vx0 = (uint32_t)x0 < (uint32_t)G.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)G.W;
    const bool vy0 = (uint32_t)y0 < (uint32_t)G.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)G.H;
    s.v[0] = vy0 && vx0; s.v[1] = vy0 && vx1; s.v[2] = vy1 && vx0; s.v[3] = vy1 && vx1;
    // modular arithmetic: a00 may wrap when x0 or y0 is -1, but only valid
    // corners keep their offset and those are in [0, image bytes)
    const uint32_t a00 = (uint32_t)y0 * G.in_line_bytes + (uint32_t)x0 * G.in_row_bytes + chan_bytes;
    s.off[0] = s.v[0] ? a00 : kOOB;
    s.off[1] = s.v[1] ? a00 + G.in_row_bytes : kOOB;
    s.off[2] = s.v[2] ? a00 + G.in_line_bytes : kOOB;
    s.off[3] = s.v[3] ? a00 + G.in_line_bytes + G.in_row_bytes : kOOB;
    return s;
}

// ---------------------------------------------------------------------------
// Forward.  T: element type; LB: bytes per gather load; NL: loads per corner
// per lane, so CPL = NL*LB/sizeof(T) channels per lane; KT: K, or 0 for a
// runtime K.
template <typename T, int LB, int NL, int KT>
__global__ __launch_bounds__(kBlock) void dcn_forward_kernel(FwdArgs a)
{
    constexpr int EPL = LB / Elem<T>::bytes;          // elements per load
    constexpr int CPL = NL * EPL;                      // channels per lane
    const Geometry& G = a.geo;
    const LaneWork lw = lane_work(G);
    if (!lw.active) return;

    const char* in_img = (const char*)a.input + (size_t)lw.n * G.in_image_bytes;
    const __amdgpu_buffer_rsrc_t rin = image_rsrc(in_img, G.in_image_bytes);
    const uint32_t chan_bytes = lw.cc * (CPL * Elem<T>::bytes);
    const size_t pix_global = (size_t)lw.n * G.Ho * G.Wo + lw.pix;
    const size_t pg = pix_global * G.groups + lw.g;
    const T* off = (const T*)a.offset + pg * G.off_stride;
    const T* mk = (const T*)a.mask + pg * G.mask_stride;
    const float bx = (float)((int)lw.wo * G.stride - G.pad + G.c0);
    const float by = (float)((int)lw.ho * G.stride - G.pad + G.c0);

    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

    auto point = [&](int i, int j, float m, float2 d) {
        const Sample s = make_sample(G, bx, by, i, j, d.x, d.y, chan_bytes);
        const float mm = s.inmap ? m : 0.f;
        const float hy = 1.0f - s.ly, hx = 1.0f - s.lx;
        const float mhy = mm * hy, mly = mm * s.ly;
        float w[4] = {mhy * hx, mhy * s.lx, mly * hx, mly * s.lx};
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = s.v[k] ? w[k] : 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                float f[EPL];
                gather<T, LB>(rin, s.off[k] + l * LB, f);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[l * EPL + e] = fmaf(w[k], f[e], acc[l * EPL + e]);
            }
        }
    };

    if constexpr (KT > 0) {
        constexpr int P = KT * KT;
        float m[P];
#pragma unroll
        for (int p = 0; p < P; ++p) m[p] = ld1(mk + p);
        if (G.softmax) {
            float mx = m[0];
#pragma unroll
            for (int p = 1; p < P; ++p) mx = fmaxf(mx, m[p]);
            float sum = 0.f;
#pragma unroll
            for (int p = 0; p < P; ++p) { m[p] = __expf(m[p] - mx); sum += m[p]; }
            const float inv = 1.0f / sum;
#pragma unroll
            for (int p = 0; p < P; ++p) m[p] *= inv;
        }
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
            for (int j = 0; j < KT; ++j) point(i, j, m[i * KT + j], ld2(off + 2 * (i * KT + j)));
    } else {
        float mx = 0.f, inv = 1.f;
        if (G.softmax) {
            mx = ld1(mk);
            for (int p = 1; p < G.P; ++p) mx = fmaxf(mx, ld1(mk + p));
            float sum = 0.f;
            for (int p = 0; p < G.P; ++p) sum += __expf(ld1(mk + p) - mx);
            inv = 1.0f / sum;
        }
        for (int i = 0; i < G.K; ++i)
            for (int j = 0; j < G.K; ++j) {
                const int p = point_of(G, i, j);
                if (p < 0) continue;
                float m = ld1(mk + p);
                if (G.softmax) m = __expf(m - mx) * inv;
                point(i, j, m, ld2(off + 2 * p));
            }
    }

    char* out = (char*)a.output + (pix_global * G.C + lw.cc * CPL) * Elem<T>::bytes;
#pragma unroll
    for (int l = 0; l < NL; ++l) store<T, LB>(out + l * LB, &acc[l * EPL]);
}

// ---------------------------------------------------------------------------
// Tiled forward.  A workgroup owns one output tile (TH x TW pixels) of one
// image and one 128-byte channel slab (the groups whose channels fall in
// that slab).  It first stages the input region those samples can reach --
// the tile's sampling centres widened by a margin ML on every side -- into
// LDS, reading each 128-byte pixel slab once with coalesced 16-byte loads;
// pixels outside the image are stored as zeros, which is exactly the zero
// padding of the definition.  Every lane then owns 32 bytes of channels of
// one output pixel (4 lanes per pixel slab) and reads its four bilinear
// corners from LDS.  A sample whose offset carries it outside the staged
// region (or a NaN coordinate) takes the global gather path instead, with
// the same off-map rules as the untiled kernel.
//
// LDS layout: region[ry][rx][128 bytes], rows of RW pixels.  Every pixel
// slab starts on bank 0, so a 16-byte read is conflict free when the 8 lanes
// served together read 8 different 16-byte slots of their (different)
// pixels.  Lanes 4k..4k+3 hold slots {0,2,4,6} of their first read; pixels
// with odd index read their two 16-byte halves in the opposite order, so the
// other four lanes of the 8 hold slots {1,3,5,7}.  The swap is undone when
// the result is stored.
constexpr int kMaxTiledTaps = 49;     // the tiled kernel serves K <= 7

struct TileGeo {
    int TH, TW;              // output tile, pixels
    int RH, RW;              // staged input region, pixels
    int ML;                  // region origin = first tile centre - ML (both axes)
    int gshift;              // log2(Cg * elem_bytes / 32): lanes per group = 1 << gshift
    int whole;               // 1: the region is the whole map plus a one-pixel border
    uint32_t tiles_x, tiles_y, slabs;
    uint32_t off_image_bytes, mask_image_bytes;   // one image of offset / mask
    float tap_x[kMaxTiledTaps];                   // (float)(i*dilation - c0) of point p
    float tap_y[kMaxTiledTaps];                   // (float)(j*dilation - c0) of point p
};

#ifndef DCN_TILE_UNROLL
#define DCN_TILE_UNROLL 1
#endif
#define DCN_PRAGMA(x) _Pragma(#x)
#define DCN_UNROLL(n) DCN_PRAGMA(unroll n)
#ifndef DCN_TILE_WAVES_PER_EU
#define DCN_TILE_WAVES_PER_EU 4   // register budget 512/4 = 128 VGPRs per lane
#endif

// floor(x) as an integer in one instruction (v_cvt_flr_i32_f32; NaN gives 0,
// +-Inf and out-of-range values saturate).
__device__ __forceinline__ int cvt_flr(float x)
{
    int r;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Neither argument is NaN.
__device__ __forceinline__ bool ordered(float x, float y)
{
    return !__builtin_isunordered(x, y);
}

// Offset pair (dx, dy) and mask value of point q of a (pixel, group), read
// through per-image buffer resources with the point in the scalar offset.
// The raw forms keep the loaded bits (one dword per offset pair for half
// types) so a prefetch of all points stays small; widen_* converts later.
template <typename T> struct RawPair { uint32_t v[Elem<T>::bytes == 4 ? 2 : 1]; };

// odd: the records may start on a 2-byte boundary (half precision, packed
// record of odd P); the pair is then read as two 16-bit halves.  The flag is
// the same for every lane of the launch.
template <typename T>
__device__ __forceinline__ RawPair<T> load_offset_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, int q, bool odd)
{
    RawPair<T> rp;
    if constexpr (Elem<T>::bytes == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, q * 8, 0);
        rp.v[0] = v[0];
        rp.v[1] = v[1];
    } else if (odd) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff, q * 4, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, voff, q * 4 + 2, 0);
        rp.v[0] = lo | (hi << 16);
    } else {
        rp.v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, q * 4, 0);
    }
    return rp;
}

template <typename T>
__device__ __forceinline__ float2 widen_pair(const RawPair<T>& rp)
{
    if constexpr (Elem<T>::bytes == 4) return make_float2(__uint_as_float(rp.v[0]), __uint_as_float(rp.v[1]));
    else return make_float2(Elem<T>::widen(rp.v[0] & 0xffffu), Elem<T>::widen(rp.v[0] >> 16));
}

template <typename T>
__device__ __forceinline__ uint32_t load_mask_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, int q)
{
    if constexpr (Elem<T>::bytes == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, q * 4, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, q * 2, 0);
}

// The whole offset record (PK pairs) and mask record (PK values) of one
// (pixel, group), fetched once with the widest loads the record's alignment
// allows: an offset record starts on a 4-byte boundary (8 for fp32), a
// half-precision mask record only on a 2-byte one.
template <typename T, int PK>
struct PointRecord {
    uint32_t off[PK * 2 * Elem<T>::bytes / 4];
    uint32_t mask[PK];
};

template <typename T, int PK>
__device__ __forceinline__ void load_record(PointRecord<T, PK>& rec, __amdgpu_buffer_rsrc_t roff, uint32_t voff,
                                            __amdgpu_buffer_rsrc_t rmk, uint32_t vmk, bool odd)
{
    constexpr int ND = PK * 2 * Elem<T>::bytes / 4;      // offset dwords
    if (Elem<T>::bytes == 2 && odd) {
        // half-precision records that may start on a 2-byte boundary (packed
        // record, odd P): read ND + 1 dwords from the dword boundary at or
        // below the record and shift each dword pair down by the misalignment.
        // The extra dword is the record's first mask value when the record is
        // dword aligned, and lies inside the record otherwise.
        const uint32_t base = voff & ~3u, sh = (voff & 2u) * 8u;
        uint32_t d[ND + 1];
        int i = 0;
#pragma unroll
        for (; i + 4 <= ND + 1; i += 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(roff, base, i * 4, 0);
            d[i] = v[0]; d[i + 1] = v[1]; d[i + 2] = v[2]; d[i + 3] = v[3];
        }
#pragma unroll
        for (; i < ND + 1; ++i) d[i] = __builtin_amdgcn_raw_buffer_load_b32(roff, base, i * 4, 0);
#pragma unroll
        for (int k = 0; k < ND; ++k) rec.off[k] = __builtin_amdgcn_alignbit(d[k + 1], d[k], sh);
    } else {
        int i = 0;
#pragma unroll
        for (; i + 4 <= ND; i += 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(roff, voff, i * 4, 0);
            rec.off[i] = v[0]; rec.off[i + 1] = v[1]; rec.off[i + 2] = v[2]; rec.off[i + 3] = v[3];
        }
#pragma unroll
        for (; i < ND; ++i) rec.off[i] = __builtin_amdgcn_raw_buffer_load_b32(roff, voff, i * 4, 0);
    }
    if constexpr (Elem<T>::bytes == 4) {
        int j = 0;
#pragma unroll
        for (; j + 4 <= PK; j += 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rmk, vmk, j * 4, 0);
            rec.mask[j] = v[0]; rec.mask[j + 1] = v[1]; rec.mask[j + 2] = v[2]; rec.mask[j + 3] = v[3];
        }
#pragma unroll
        for (; j < PK; ++j) rec.mask[j] = __builtin_amdgcn_raw_buffer_load_b32(rmk, vmk, j * 4, 0);
    } else {
        // PK half values from a 2-byte boundary: read the dwords that hold
        // them (from the dword boundary at or below, so byte offsets must be
        // true to the address's alignment, see record_rsrc) and shift each
        // dword pair down by the misalignment.  Every dword read holds a byte
        // of the record, except the last one of an even PK on a dword
        // boundary, which is then not read.
        constexpr int MW = PK / 2 + 1;
        const uint32_t mb = vmk & ~3u, msh = (vmk & 2u) * 8u;
        uint32_t md[MW];
        int k = 0;
#pragma unroll
        for (; k + 4 <= MW - 1; k += 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rmk, mb, k * 4, 0);
            md[k] = v[0]; md[k + 1] = v[1]; md[k + 2] = v[2]; md[k + 3] = v[3];
        }
#pragma unroll
        for (; k < MW - 1; ++k) md[k] = __builtin_amdgcn_raw_buffer_load_b32(rmk, mb, k * 4, 0);
        if constexpr (PK % 2 == 1) md[MW - 1] = __builtin_amdgcn_raw_buffer_load_b32(rmk, mb, (MW - 1) * 4, 0);
        else md[MW - 1] = msh ? __builtin_amdgcn_raw_buffer_load_b32(rmk, mb, (MW - 1) * 4, 0) : 0u;
#pragma unroll
        for (int j = 0; j < PK; ++j) {
            const uint32_t w = __builtin_amdgcn_alignbit(md[j / 2 + 1], md[j / 2], msh);
            rec.mask[j] = (j & 1) ? (w >> 16) : (w & 0xffffu);
        }
    }
}

template <typename T, int PK>
__device__ __forceinline__ float2 record_pair(const PointRecord<T, PK>& rec, int q)
{
    if constexpr (Elem<T>::bytes == 4) return make_float2(__uint_as_float(rec.off[2 * q]), __uint_as_float(rec.off[2 * q + 1]));
    else return make_float2(Elem<T>::widen(rec.off[q] & 0xffffu), Elem<T>::widen(rec.off[q] >> 16));
}

template <typename T>
__device__ __forceinline__ float2 load_offset_pair(__amdgpu_buffer_rsrc_t r, uint32_t voff, int q)
{
    if constexpr (Elem<T>::bytes == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, q * 8, 0);
        return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
    } else {
        // two 16-bit reads: the record may start on a 2-byte boundary (ld2)
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff, q * 4, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, voff, q * 4 + 2, 0);
        return make_float2(Elem<T>::widen(lo), Elem<T>::widen(hi));
    }
}

template <typename T>
__device__ __forceinline__ float load_mask_value(__amdgpu_buffer_rsrc_t r, uint32_t voff, int q)
{
    if constexpr (Elem<T>::bytes == 4)
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, q * 4, 0));
    else
        return Elem<T>::widen(__builtin_amdgcn_raw_buffer_load_b16(r, voff, q * 2, 0));
}

// One sampling point of the tiled kernel: its four corner rows (8 dwords
// each, this lane's 32 bytes) and its modulated bilinear weights.
struct TiledPoint {
    uint32_t raw[4][8];
    float w[4];
};

// Per-lane constants of the tiled kernel's compute phase.
struct TiledLane {
    float bx, by;                 // sampling centre (absolute input coordinates)
    int x_lo, y_lo;               // staged region origin
    uint32_t xlim, ylim;          // RW-1, RH-1
    uint32_t lane_first;          // this lane's first 16-byte slot in a pixel slab
    uint32_t RW, RWB;             // region width in pixels and in bytes
    uint32_t gl_first, gl_second; // the two halves inside an input pixel row
};

// Coordinates, weights and corner reads of one point: from the staged region
// when all four corners lie inside it, else gathered from global memory with
// the untiled kernel's off-map rules.  xt, yt: the tap's part of the
// coordinates, fmaf(alpha, tap, base).
template <typename T>
__device__ __forceinline__ TiledPoint tiled_fetch(const Geometry& G, const TiledLane& L, const char* lds,
                                                  __amdgpu_buffer_rsrc_t rin, float xt, float yt,
                                                  float2 d, float m)
{
    TiledPoint pt;
    const float x = fmaf(G.alpha, d.x, xt);
    const float y = fmaf(G.alpha, d.y, yt);
    // Floor and fraction come from the absolute coordinate (x - x_lo is not
    // exact when x_lo < 0); the region test is on the integer floor.
    // cvt_flr saturates +-Inf to out-of-range values; NaN is rejected by the
    // ordered compare.
    const uint32_t ix = (uint32_t)(cvt_flr(x) - L.x_lo), iy = (uint32_t)(cvt_flr(y) - L.y_lo);
    float lx, ly, mm = m;
    if ((ix < L.xlim) & (iy < L.ylim) & ordered(x, y)) {
        lx = __builtin_amdgcn_fractf(x);
        ly = __builtin_amdgcn_fractf(y);
        const uint32_t a0 = (__umul24(iy, L.RW) + ix) * 128u + L.lane_first;
        const uint32_t a1 = a0 ^ 16u;
        const uint32_t ca[4] = {0u, 128u, L.RWB, L.RWB + 128u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 v0 = *(const uint4*)(lds + a0 + ca[k]);
            const uint4 v1 = *(const uint4*)(lds + a1 + ca[k]);
            pt.raw[k][0] = v0.x; pt.raw[k][1] = v0.y; pt.raw[k][2] = v0.z; pt.raw[k][3] = v0.w;
            pt.raw[k][4] = v1.x; pt.raw[k][5] = v1.y; pt.raw[k][6] = v1.z; pt.raw[k][7] = v1.w;
        }
    } else {
        // outside the staged region: gather from memory, or nothing at all
        // for a sample with no corner on the map (or a NaN coordinate)
        float fx = floorf(x), fy = floorf(y);
        lx = x - fx;
        ly = y - fy;
        const bool inmap = x > -1.0f && x < (float)G.W && y > -1.0f && y < (float)G.H;
        if (!inmap) { fx = -2.0f; fy = -2.0f; lx = 0.f; ly = 0.f; mm = 0.f; }
        const int x0 = (int)fx, y0 = (int)fy;
        const bool vx0 = (uint32_t)x0 < (uint32_t)G.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)G.W;
        const bool vy0 = (uint32_t)y0 < (uint32_t)G.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)G.H;
        const bool vk[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
        const uint32_t a00 = (uint32_t)y0 * G.in_line_bytes + (uint32_t)x0 * G.in_row_bytes;
        const uint32_t ck[4] = {0u, G.in_row_bytes, G.in_line_bytes, G.in_line_bytes + G.in_row_bytes};
        if (inmap) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t o0 = vk[k] ? a00 + ck[k] + L.gl_first : kOOB;
                const uint32_t o1 = vk[k] ? a00 + ck[k] + L.gl_second : kOOB;
                const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rin, o0, 0, 0);
                const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rin, o1, 0, 0);
                pt.raw[k][0] = v0[0]; pt.raw[k][1] = v0[1]; pt.raw[k][2] = v0[2]; pt.raw[k][3] = v0[3];
                pt.raw[k][4] = v1[0]; pt.raw[k][5] = v1[1]; pt.raw[k][6] = v1[2]; pt.raw[k][7] = v1[3];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int c = 0; c < 8; ++c) pt.raw[k][c] = 0u;
        }
    }
    // bilinear weights with the modulation folded in; each is formed with
    // relative error <= 2 ulp (the one-minus factors are fused, so a weight
    // near zero is not the difference of two rounded values)
    const float mly = mm * ly, mhy = fmaf(-mm, ly, mm);
    pt.w[0] = fmaf(-mhy, lx, mhy);
    pt.w[1] = mhy * lx;
    pt.w[2] = fmaf(-mly, lx, mly);
    pt.w[3] = mly * lx;
    return pt;
}

// tiled_fetch for a region holding the whole map, a one-pixel zero border
// and one more zero row (origin -1, -1; rows H and H + 1 are zero): every
// sample with a corner on the map is inside it, and any other sample (or a
// NaN coordinate) reads the 2x2 block of zeros at the bottom-left with zero
// weights.  No branch, no gather from memory.
template <typename T>
__device__ __forceinline__ TiledPoint whole_fetch(const Geometry& G, const TiledLane& L, const char* lds, float xt,
                                                  float yt, float2 d, float m)
{
    TiledPoint pt;
    const float x = fmaf(G.alpha, d.x, xt);
    const float y = fmaf(G.alpha, d.y, yt);
    const bool inmap = x > -1.0f && x < (float)G.W && y > -1.0f && y < (float)G.H;
    const uint32_t ix = inmap ? (uint32_t)(cvt_flr(x) + 1) : 0u;
    const uint32_t iy = inmap ? (uint32_t)(cvt_flr(y) + 1) : (uint32_t)(G.H + 1);
    const float lx = inmap ? __builtin_amdgcn_fractf(x) : 0.f, ly = inmap ? __builtin_amdgcn_fractf(y) : 0.f;
    const float mm = inmap ? m : 0.f;
    const uint32_t a0 = (__umul24(iy, L.RW) + ix) * 128u + L.lane_first;
    const uint32_t a1 = a0 ^ 16u;
    const uint32_t ca[4] = {0u, 128u, L.RWB, L.RWB + 128u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 v0 = *(const uint4*)(lds + a0 + ca[k]);
        const uint4 v1 = *(const uint4*)(lds + a1 + ca[k]);
        pt.raw[k][0] = v0.x; pt.raw[k][1] = v0.y; pt.raw[k][2] = v0.z; pt.raw[k][3] = v0.w;
        pt.raw[k][4] = v1.x; pt.raw[k][5] = v1.y; pt.raw[k][6] = v1.z; pt.raw[k][7] = v1.w;
    }
    const float mly = mm * ly, mhy = fmaf(-mm, ly, mm);
    pt.w[0] = fmaf(-mhy, lx, mhy);
    pt.w[1] = mhy * lx;
    pt.w[2] = fmaf(-mly, lx, mly);
    pt.w[3] = mly * lx;
    return pt;
}

template <typename T, int CPL>
__device__ __forceinline__ void tiled_accumulate(const TiledPoint& pt, float* acc)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (Elem<T>::bytes == 4) {
                acc[c] = fmaf(pt.w[k], __uint_as_float(pt.raw[k][c]), acc[c]);
            } else {
                acc[2 * c] = fmaf(pt.w[k], Elem<T>::widen(pt.raw[k][c] & 0xffffu), acc[2 * c]);
                acc[2 * c + 1] = fmaf(pt.w[k], Elem<T>::widen(pt.raw[k][c] >> 16), acc[2 * c + 1]);
            }
        }
    }
}

// Image, slab and region origin of one tile (wave-uniform values).
struct TileCoord {
    uint32_t n, slab;
    int ho0, wo0, y_lo, x_lo;
};

__device__ __forceinline__ TileCoord tile_coord(const Geometry& G, const TileGeo& tg, uint32_t tile)
{
    TileCoord c;
    uint32_t rest = tile;
    const uint32_t tx = rest % tg.tiles_x;
    rest /= tg.tiles_x;
    const uint32_t ty = rest % tg.tiles_y;
    rest /= tg.tiles_y;
    c.slab = rest % tg.slabs;
    c.n = rest / tg.slabs;
    c.ho0 = (int)ty * tg.TH;
    c.wo0 = (int)tx * tg.TW;
    // A region cut down to the map and a one-pixel border starts no earlier
    // than -1: rows and columns before it hold nothing a sample on the map
    // can read.
    const int y_lo = c.ho0 * G.stride - G.pad + G.c0 - tg.ML;
    const int x_lo = c.wo0 * G.stride - G.pad + G.c0 - tg.ML;
    c.y_lo = tg.whole ? -1 : ((tg.RH == G.H + 2 && y_lo < -1) ? -1 : y_lo);   // whole: RH = H + 3
    c.x_lo = tg.whole ? -1 : ((tg.RW == G.W + 2 && x_lo < -1) ? -1 : x_lo);
    return c;
}

// Stage region rows [r0, r1) of tile c into buf with LDS-direct buffer loads
// (asynchronous, no registers): lane t copies 16-byte chunk e of each row;
// the 64 lanes of a wave fill 1 KB of LDS contiguously (lane l at base +
// 16*l).  Off-image pixels get an out-of-range offset and are written as
// zeros, which is the zero padding of the definition.  Rows above and below
// the image (a range every lane shares) use that offset outright; on image
// rows a lane steps its offset by one image row.
template <int NT>
__device__ __forceinline__ void stage_rows(const Geometry& G, const TileGeo& tg, const void* input,
                                           const TileCoord& c, uint4* buf, int r0, int r1, int t)
{
    const int RW8 = tg.RW * 8;
    const __amdgpu_buffer_rsrc_t rin =
        image_rsrc((const char*)input + (size_t)c.n * G.in_image_bytes, G.in_image_bytes);
    // image rows are region rows [ra, rb)
    const int ra = -c.y_lo < r0 ? r0 : (-c.y_lo > r1 ? r1 : -c.y_lo);
    const int rb = G.H - c.y_lo < ra ? ra : (G.H - c.y_lo > r1 ? r1 : G.H - c.y_lo);
    for (int e = t; e < RW8; e += NT) {
        const int gx = c.x_lo + (e >> 3);
        const bool col_ok = (uint32_t)gx < (uint32_t)G.W;
        uint4* wave_dst = buf + (e & ~63);
        for (int ry = r0; ry < ra; ++ry)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rin, (__attribute__((address_space(3))) void*)(wave_dst + ry * RW8), 16, kOOB, 0, 0, 0);
        uint32_t off = col_ok ? (uint32_t)(c.y_lo + ra) * G.in_line_bytes + (uint32_t)gx * G.in_row_bytes +
                                    c.slab * 128u + (uint32_t)(e & 7) * 16u
                              : kOOB;
        const uint32_t step = col_ok ? G.in_line_bytes : 0u;
        for (int ry = ra; ry < rb; ++ry) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rin, (__attribute__((address_space(3))) void*)(wave_dst + ry * RW8), 16, off, 0, 0, 0);
            off += step;
        }
        for (int ry = rb; ry < r1; ++ry)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rin, (__attribute__((address_space(3))) void*)(wave_dst + ry * RW8), 16, kOOB, 0, 0, 0);
    }
}

// Tiled forward: a workgroup stages the input region of one output tile into
// LDS, then each lane accumulates 32 bytes of channels of one output pixel.
// The lane's offset/mask record is requested before the wait for the region,
// so the two memory latencies overlap.
// GATE: the DCNv4 layer's centre-feature gate in the epilogue, out = y (1 - s)
// + v s with y the sampled result, v the input at the output pixel itself (in
// the staged region: stride 1, taps centred on the pixel) and s the sigmoid
// of the (pixel, group)'s logit; y may also be stored before the gate.
template <typename T, int KT, int NT, bool SOFTMAX, bool WHOLE, bool GATE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DCN_TILE_WAVES_PER_EU)))
void dcn_forward_tiled(FwdArgs a, TileGeo tg)
{
    constexpr int EB = Elem<T>::bytes;
    constexpr int CPL = 32 / EB;        // channels per lane
    constexpr int EPR = 16 / EB;        // elements per 16-byte read
    extern __shared__ uint4 region[];
    const Geometry& G = a.geo;
    const int t = threadIdx.x;

    const TileCoord cur = tile_coord(G, tg, xcd_remap(blockIdx.x, gridDim.x));
    stage_rows<NT>(G, tg, a.input, cur, region, 0, tg.RH, t);

    // ---- this lane: 32 bytes of channels of one output pixel of the tile
    const int p = t >> 2, sub = t & 3;
    const int py = p / tg.TW, px = p - py * tg.TW;
    const int P = KT > 0 ? KT * KT : G.P;
    const int swp = p & 1;                       // read order of the two halves
    TiledLane L;
    L.xlim = (uint32_t)(tg.RW - 1);
    L.ylim = (uint32_t)(tg.RH - 1);
    L.lane_first = (uint32_t)sub * 32u + (uint32_t)swp * 16u;
    L.RW = (uint32_t)tg.RW;
    L.RWB = (uint32_t)tg.RW * 128u;
    const int ho = cur.ho0 + py, wo = cur.wo0 + px;
    const bool active = p < tg.TH * tg.TW && ho < G.Ho && wo < G.Wo;
    const uint32_t g = cur.slab * (4u >> tg.gshift) + ((uint32_t)sub >> tg.gshift);
    const uint32_t pg_img = active ? ((uint32_t)ho * (uint32_t)G.Wo + (uint32_t)wo) * (uint32_t)G.groups + g : 0u;
    const __amdgpu_buffer_rsrc_t rin =
        image_rsrc((const char*)a.input + (size_t)cur.n * G.in_image_bytes, G.in_image_bytes);
    const RecordRsrc ro =
        record_rsrc((const char*)a.offset + (size_t)cur.n * tg.off_image_bytes, tg.off_image_bytes);
    const __amdgpu_buffer_rsrc_t roff = ro.r;
    const RecordRsrc rm =
        record_rsrc((const char*)a.mask + (size_t)cur.n * tg.mask_image_bytes, tg.mask_image_bytes);
    const __amdgpu_buffer_rsrc_t rmk = rm.r;
    const uint32_t voff = pg_img * (uint32_t)(G.off_stride * EB) + ro.lead;
    const bool odd = EB == 2 && (G.off_stride & 1);   // records on 2-byte boundaries
    const uint32_t vmk = pg_img * (uint32_t)(G.mask_stride * EB) + rm.lead;
    L.bx = (float)(wo * G.stride - G.pad + G.c0);
    L.by = (float)(ho * G.stride - G.pad + G.c0);
    L.x_lo = cur.x_lo;
    L.y_lo = cur.y_lo;
    L.gl_first = cur.slab * 128u + L.lane_first;
    L.gl_second = L.gl_first ^ 16u;
    const char* lds = (const char*)region;

    auto mval = [&](uint32_t raw) {
        return Elem<T>::bytes == 4 ? __uint_as_float(raw) : Elem<T>::widen(raw);
    };
    float zval = 0.f;
    if constexpr (GATE) {
        // the gate logit, in flight with the record and the region
        if (active) zval = ld1((const T*)a.gate + (size_t)cur.n * G.Ho * G.Wo * G.groups + pg_img);
    }
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

    if constexpr (KT > 0) {
        // K fixed: the (pixel, group)'s offset and mask records come in once
        // (a per-point load would re-touch the same cache lines P times)
        // and the points are unrolled so the record stays in registers.
        constexpr int PK = KT * KT;
        PointRecord<T, PK> rec;
        load_record<T, PK>(rec, roff, voff, rmk, vmk, odd);
        __builtin_amdgcn_s_waitcnt(0);   // the region (and the record) have landed
        __syncthreads();
        float mx = 0.f, inv = 1.f;
        if constexpr (SOFTMAX) {
            mx = mval(rec.mask[0]);
#pragma unroll
            for (int q = 1; q < PK; ++q) mx = fmaxf(mx, mval(rec.mask[q]));
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < PK; ++q) sum += __expf(mval(rec.mask[q]) - mx);
            inv = 1.0f / sum;
        }
        // the taps' part of the coordinates, once per column and row of taps
        float xt[KT], yt[KT];
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            xt[i] = fmaf(G.alpha, tg.tap_x[i * KT], L.bx);
            yt[i] = fmaf(G.alpha, tg.tap_y[i], L.by);
        }
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            if (active) {
                float m = mval(rec.mask[q]);
                if constexpr (SOFTMAX) m = __expf(m - mx) * inv;
                const TiledPoint pt =
                    WHOLE ? whole_fetch<T>(G, L, lds, xt[q / KT], yt[q % KT], record_pair<T, PK>(rec, q), m)
                          : tiled_fetch<T>(G, L, lds, rin, xt[q / KT], yt[q % KT], record_pair<T, PK>(rec, q), m);
                tiled_accumulate<T, CPL>(pt, acc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        __builtin_amdgcn_s_waitcnt(0);   // the region has landed
        __syncthreads();
        float mx = 0.f, inv = 1.f;
        if constexpr (SOFTMAX) {
            mx = load_mask_value<T>(rmk, vmk, 0);
            for (int q = 1; q < P; ++q) mx = fmaxf(mx, load_mask_value<T>(rmk, vmk, q));
            float sum = 0.f;
            for (int q = 0; q < P; ++q) sum += __expf(load_mask_value<T>(rmk, vmk, q) - mx);
            inv = 1.0f / sum;
        }
        auto fetch = [&](int q, const RawPair<T>& d, uint32_t mraw) {
            float m = mval(mraw);
            if constexpr (SOFTMAX) m = __expf(m - mx) * inv;
            const float xt = fmaf(G.alpha, tg.tap_x[q], L.bx), yt = fmaf(G.alpha, tg.tap_y[q], L.by);
            return WHOLE ? whole_fetch<T>(G, L, lds, xt, yt, widen_pair<T>(d), m)
                         : tiled_fetch<T>(G, L, lds, rin, xt, yt, widen_pair<T>(d), m);
        };

        // Software pipeline over the points, two per (rolled) iteration: the
        // corner reads of point q+1 are in flight while point q accumulates,
        // and each point's offsets and mask are requested two points ahead.
        // Rolled, the compiler cannot hoist further points' reads and run
        // out of registers.
        RawPair<T> dA, dB;
        uint32_t mA = 0u, mB = 0u;
        dA = load_offset_raw<T>(roff, voff, 0, odd);
        mA = load_mask_raw<T>(rmk, vmk, 0);
        if (P > 1) { dB = load_offset_raw<T>(roff, voff, 1, odd); mB = load_mask_raw<T>(rmk, vmk, 1); }
        TiledPoint ptA, ptB;
        if (active) ptA = fetch(0, dA, mA);
        if (P > 2) { dA = load_offset_raw<T>(roff, voff, 2, odd); mA = load_mask_raw<T>(rmk, vmk, 2); }
        int q = 0;
        DCN_UNROLL(1)
        for (; q + 1 < P; q += 2) {
            // here: ptA = point q (reads issued), dB = point q+1, dA = point q+2
            if (active) ptB = fetch(q + 1, dB, mB);
            if (q + 3 < P) { dB = load_offset_raw<T>(roff, voff, q + 3, odd); mB = load_mask_raw<T>(rmk, vmk, q + 3); }
            if (active) tiled_accumulate<T, CPL>(ptA, acc);
            if (q + 2 < P) {
                if (active) ptA = fetch(q + 2, dA, mA);
                if (q + 4 < P) { dA = load_offset_raw<T>(roff, voff, q + 4, odd); mA = load_mask_raw<T>(rmk, vmk, q + 4); }
            }
            if (active) tiled_accumulate<T, CPL>(ptB, acc);
        }
        if (q < P) {   // odd number of points: the last one is in ptA
            if (active) tiled_accumulate<T, CPL>(ptA, acc);
        }
    }

    if (active) {
        // store the lane's 32 bytes, undoing the half swap
        const size_t at = ((size_t)cur.n * G.Ho * G.Wo + (size_t)ho * G.Wo + wo) * G.C * EB + cur.slab * 128u +
                          (uint32_t)sub * 32u;
        if constexpr (GATE) {
            if (a.core_out) {
                char* co = (char*)a.core_out + at;
                store<T, 16>(co + swp * 16, &acc[0]);
                store<T, 16>(co + (swp ^ 1) * 16, &acc[EPR]);
            }
            // the output pixel's own input row, read in the lane's order
            const GateWeights gw = gate_weights(zval);
            const uint32_t ac = ((uint32_t)(ho - L.y_lo) * L.RW + (uint32_t)(wo - L.x_lo)) * 128u + L.lane_first;
            const uint4 v0 = *(const uint4*)(lds + ac);
            const uint4 v1 = *(const uint4*)(lds + (ac ^ 16u));
            const uint32_t cv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if constexpr (EB == 4) {
                    acc[c] = fmaf(gw.s, __uint_as_float(cv[c]), gw.t * acc[c]);
                } else {
                    acc[2 * c] = fmaf(gw.s, Elem<T>::widen(cv[c] & 0xffffu), gw.t * acc[2 * c]);
                    acc[2 * c + 1] = fmaf(gw.s, Elem<T>::widen(cv[c] >> 16), gw.t * acc[2 * c + 1]);
                }
            }
        }
        char* out = (char*)a.output + at;
        store<T, 16>(out + swp * 16, &acc[0]);
        store<T, 16>(out + (swp ^ 1) * 16, &acc[EPR]);
    }
}

// ---------------------------------------------------------------------------
// Backward (binary32).  Same lane mapping; L = Cg/CPL lanes per group, a
// power of two.  Per point and corner k each lane forms
// s_k = sum over its channels of g_c * f_kc; then
//   gm  = sum_k w_k s_k,   gdx = sum_k (dw_k/dx) s_k,   gdy = sum_k (dw_k/dy) s_k
// are summed over the L lanes of the group with cross-lane adds, and every
// valid corner receives grad_input[corner, c] += m * w_k * g_c as a float
// atomic (performed at L2).  For the softmax case grad_mask is finished in a
// second pass over P that rereads the raw gm_p this same lane stored.
template <int L>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int LB, int L, int KT>
__global__ __launch_bounds__(kBlock) void dcn_backward_kernel(BwdArgs a)
{
    constexpr int CPL = LB / 4;
    const Geometry& G = a.geo;
    const LaneWork lw = lane_work(G);
    // Inactive lanes (past the image) stay for the cross-lane sums but touch
    // no memory; a group is always wholly active or wholly inactive.
    const bool act = lw.active;

    const char* in_img = (const char*)a.input + (size_t)lw.n * G.in_image_bytes;
    const __amdgpu_buffer_rsrc_t rin = image_rsrc(in_img, G.in_image_bytes);
    const uint32_t chan_bytes = lw.cc * (CPL * 4);
    const size_t pix_global = (size_t)lw.n * G.Ho * G.Wo + lw.pix;
    const size_t pg = pix_global * G.groups + lw.g;
    const float* off = (const float*)a.offset + pg * G.off_stride;
    const float* mk = (const float*)a.mask + pg * G.mask_stride;
    float* goff = (float*)a.grad_offset + pg * G.off_stride;
    float* gmk = (float*)a.grad_mask + pg * G.mask_stride;
    char* gin = (char*)a.grad_input + (size_t)lw.n * G.in_image_bytes;
    const int bxi = (int)lw.wo * G.stride - G.pad + G.c0;
    const int byi = (int)lw.ho * G.stride - G.pad + G.c0;
    const float bx = (float)bxi, by = (float)byi;
    const bool leader = (lw.cc & (L - 1)) == 0;

    float go[CPL];
    {
        const float* gp = (const float*)a.grad_out + pix_global * G.C + lw.cc * CPL;
#pragma unroll
        for (int c = 0; c < CPL; ++c) go[c] = act ? gp[c] : 0.f;
    }

    float mx = 0.f, inv = 1.f;
    if (G.softmax && act) {
        mx = mk[0];
        for (int p = 1; p < G.P; ++p) mx = fmaxf(mx, mk[p]);
        float sum = 0.f;
        for (int p = 0; p < G.P; ++p) sum += __expf(mk[p] - mx);
        inv = 1.0f / sum;
    }
    float dot = 0.f;   // sum_q m_q gm_q (softmax)

    const int K = KT > 0 ? KT : G.K;
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < K; ++j) {
            const int p = point_of(G, i, j);
            if (p < 0) continue;                                // (the same for every lane)
            float m = 0.f;
            float2 d = make_float2(__builtin_nanf(""), 0.f);   // inactive: never on the map
            if (act) {
                m = mk[p];
                if (G.softmax) m = __expf(m - mx) * inv;
                d = ld2(off + 2 * p);
            }
            const Sample s = make_sample(G, bx, by, i, j, d.x, d.y, chan_bytes);
            const float hy = 1.0f - s.ly, hx = 1.0f - s.lx;
            const float wb[4] = {hy * hx, hy * s.lx, s.ly * hx, s.ly * s.lx};
            const float dwx[4] = {-hy, hy, -s.ly, s.ly};
            const float dwy[4] = {-hx, -s.lx, hx, s.lx};
            float gm = 0.f, gdx = 0.f, gdy = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float f[CPL];
                gather<float, LB>(rin, s.off[k], f);
                float sk = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) sk = fmaf(go[c], f[c], sk);
                gm = fmaf(wb[k], sk, gm);
                gdx = fmaf(dwx[k], sk, gdx);
                gdy = fmaf(dwy[k], sk, gdy);
                // corners near the sampling base were added by the owner kernel
                const bool near = a.near_m >= 0 &&
                                  (uint32_t)(s.x0 + (k & 1) - bxi + a.near_m) <= 2u * (uint32_t)a.near_m &&
                                  (uint32_t)(s.y0 + (k >> 1) - byi + a.near_m) <= 2u * (uint32_t)a.near_m;
                if (s.v[k] && !near) {
                    const float mw = m * wb[k];
                    float* dst = (float*)(gin + s.off[k]);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) atomicAdd(dst + c, mw * go[c]);
                }
            }
            gm = group_sum<L>(gm);
            gdx = group_sum<L>(gdx);
            gdy = group_sum<L>(gdy);
            if (!s.inmap) { gm = 0.f; gdx = 0.f; gdy = 0.f; }
            if (act && leader) {
                *(float2*)(goff + 2 * p) = make_float2(G.alpha * m * gdx, G.alpha * m * gdy);
                gmk[p] = gm;
            }
            dot = fmaf(m, gm, dot);
        }
    if (G.softmax && act && leader) {
        for (int p = 0; p < G.P; ++p) {
            const float m = __expf(mk[p] - mx) * inv;
            gmk[p] = m * (gmk[p] - dot);
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled gradient kernel (binary32): grad_offset and grad_mask, plus the
// atomic adds of corners that are not near their sample's base (the owner
// kernel has written every near one).  The input region of an output tile is
// staged in LDS exactly as for the forward; a lane owns 8 channels of one
// output pixel, reads its corners from the region (or, outside it, from
// global memory), and the lanes of a group sum their partial dot products
// with cross-lane shuffles.
struct GradPoint {
    uint32_t raw[4][8];
    float lx, ly;
    int x0, y0;
    bool inmap;
};

__device__ __forceinline__ GradPoint tiled_fetch_grad(const Geometry& G, const TiledLane& L, const char* lds,
                                                      __amdgpu_buffer_rsrc_t rin, float tapx, float tapy, float2 d)
{
    GradPoint pt;
    const float x = fmaf(G.alpha, d.x, fmaf(G.alpha, tapx, L.bx));
    const float y = fmaf(G.alpha, d.y, fmaf(G.alpha, tapy, L.by));
    // the skip rule of the definition (false for NaN)
    pt.inmap = x > -1.0f && x < (float)G.W && y > -1.0f && y < (float)G.H;
    const float fx = floorf(x), fy = floorf(y);
    pt.x0 = (int)fx;
    pt.y0 = (int)fy;
    pt.lx = x - fx;
    pt.ly = y - fy;
    const uint32_t ix = (uint32_t)(pt.x0 - L.x_lo), iy = (uint32_t)(pt.y0 - L.y_lo);
    if ((ix < L.xlim) & (iy < L.ylim) & pt.inmap) {
        const uint32_t a0 = (__umul24(iy, L.RW) + ix) * 128u + L.lane_first;
        const uint32_t a1 = a0 ^ 16u;
        const uint32_t ca[4] = {0u, 128u, L.RWB, L.RWB + 128u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 v0 = *(const uint4*)(lds + a0 + ca[k]);
            const uint4 v1 = *(const uint4*)(lds + a1 + ca[k]);
            pt.raw[k][0] = v0.x; pt.raw[k][1] = v0.y; pt.raw[k][2] = v0.z; pt.raw[k][3] = v0.w;
            pt.raw[k][4] = v1.x; pt.raw[k][5] = v1.y; pt.raw[k][6] = v1.z; pt.raw[k][7] = v1.w;
        }
    } else {
        const int x0 = pt.inmap ? pt.x0 : -2, y0 = pt.inmap ? pt.y0 : -2;
        const bool vx0 = (uint32_t)x0 < (uint32_t)G.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)G.W;
        const bool vy0 = (uint32_t)y0 < (uint32_t)G.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)G.H;
        const bool vk[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
        const uint32_t a00 = (uint32_t)y0 * G.in_line_bytes + (uint32_t)x0 * G.in_row_bytes;
        const uint32_t ck[4] = {0u, G.in_row_bytes, G.in_line_bytes, G.in_line_bytes + G.in_row_bytes};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t o0 = vk[k] ? a00 + ck[k] + L.gl_first : kOOB;
            const uint32_t o1 = vk[k] ? a00 + ck[k] + L.gl_second : kOOB;
            const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rin, o0, 0, 0);
            const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rin, o1, 0, 0);
            pt.raw[k][0] = v0[0]; pt.raw[k][1] = v0[1]; pt.raw[k][2] = v0[2]; pt.raw[k][3] = v0[3];
            pt.raw[k][4] = v1[0]; pt.raw[k][5] = v1[1]; pt.raw[k][6] = v1[2]; pt.raw[k][7] = v1[3];
        }
    }
    return pt;
}

// Sums over lanes l ^ 1 and l ^ 2 within a quad of lanes (DPP quad permutes).
__device__ __forceinline__ float quad_xor1(float v)
{
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v)
{
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Packed atomic add of two adjacent half-precision elements (each add rounds
// once to the dtype).
template <typename T>
__device__ __forceinline__ void atomic_add_pair(void* p, float x, float y)
{
    if constexpr (std::is_same<T, _Float16>::value) {
        typedef _Float16 v2 __attribute__((ext_vector_type(2)));
        const v2 v = {(_Float16)x, (_Float16)y};
        __builtin_amdgcn_global_atomic_fadd_v2f16((__attribute__((address_space(1))) v2*)p, v);
    } else {
        typedef __bf16 v2 __attribute__((ext_vector_type(2)));
        const v2 v = {(__bf16)x, (__bf16)y};
        __builtin_amdgcn_global_atomic_fadd_v2bf16((__attribute__((address_space(1))) v2*)p, v);
    }
}

template <typename T, int KT, int NT, bool SOFTMAX>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DCN_TILE_WAVES_PER_EU)))
void dcn_backward_grad_tiled(BwdArgs a, TileGeo tg)
{
    constexpr int EB = Elem<T>::bytes;
    constexpr int CPL = 32 / EB;        // channels per lane
    extern __shared__ uint4 region[];
    const Geometry& G = a.geo;
    const int t = threadIdx.x;
    const TileCoord cur = tile_coord(G, tg, xcd_remap(blockIdx.x, gridDim.x));
    stage_rows<NT>(G, tg, a.input, cur, region, 0, tg.RH, t);

    const int p = t >> 2, sub = t & 3;
    const int py = p / tg.TW, px = p - py * tg.TW;
    const int P = KT > 0 ? KT * KT : G.P;
    const int swp = p & 1;
    TiledLane L;
    L.xlim = (uint32_t)(tg.RW - 1);
    L.ylim = (uint32_t)(tg.RH - 1);
    L.lane_first = (uint32_t)sub * 32u + (uint32_t)swp * 16u;
    L.RW = (uint32_t)tg.RW;
    L.RWB = (uint32_t)tg.RW * 128u;
    const int ho = cur.ho0 + py, wo = cur.wo0 + px;
    const bool active = p < tg.TH * tg.TW && ho < G.Ho && wo < G.Wo;
    const uint32_t g = cur.slab * (4u >> tg.gshift) + ((uint32_t)sub >> tg.gshift);
    const bool leader = (sub & ((1 << tg.gshift) - 1)) == 0;
    const uint32_t pg_img = active ? ((uint32_t)ho * (uint32_t)G.Wo + (uint32_t)wo) * (uint32_t)G.groups + g : 0u;
    const __amdgpu_buffer_rsrc_t rin =
        image_rsrc((const char*)a.input + (size_t)cur.n * G.in_image_bytes, G.in_image_bytes);
    const RecordRsrc ro =
        record_rsrc((const char*)a.offset + (size_t)cur.n * tg.off_image_bytes, tg.off_image_bytes);
    const __amdgpu_buffer_rsrc_t roff = ro.r;
    const RecordRsrc rm =
        record_rsrc((const char*)a.mask + (size_t)cur.n * tg.mask_image_bytes, tg.mask_image_bytes);
    const __amdgpu_buffer_rsrc_t rmk = rm.r;
    const uint32_t voff = pg_img * (uint32_t)(G.off_stride * EB) + ro.lead;
    const bool odd = EB == 2 && (G.off_stride & 1);   // records on 2-byte boundaries
    const uint32_t vmk = pg_img * (uint32_t)(G.mask_stride * EB) + rm.lead;
    const int bxi = wo * G.stride - G.pad + G.c0, byi = ho * G.stride - G.pad + G.c0;
    L.bx = (float)bxi;
    L.by = (float)byi;
    L.x_lo = cur.x_lo;
    L.y_lo = cur.y_lo;
    L.gl_first = cur.slab * 128u + L.lane_first;
    L.gl_second = L.gl_first ^ 16u;
    const uint32_t M2 = 2u * (uint32_t)a.near_m;

    // upstream gradient of this lane's channels, in the order its corner reads arrive
    float go[CPL];
    const size_t pix = ((size_t)cur.n * G.Ho + (size_t)ho) * G.Wo + wo;
    char* gin = (char*)a.grad_input + (size_t)cur.n * G.in_image_bytes;
    T* goff = (T*)a.grad_offset + ((size_t)cur.n * G.Ho * G.Wo * G.groups + pg_img) * G.off_stride;
    T* gmk = (T*)a.grad_mask + ((size_t)cur.n * G.Ho * G.Wo * G.groups + pg_img) * G.mask_stride;
    if (active) {
        const char* gp = (const char*)a.grad_out + pix * G.C * EB + cur.slab * 128u + (uint32_t)sub * 32u;
        const uint4 h0 = *(const uint4*)(gp + swp * 16), h1 = *(const uint4*)(gp + (swp ^ 1) * 16);
        const uint32_t w[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (EB == 4) {
                go[c] = __uint_as_float(w[c]);
            } else {
                go[2 * c] = Elem<T>::widen(w[c] & 0xffffu);
                go[2 * c + 1] = Elem<T>::widen(w[c] >> 16);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) go[c] = 0.f;
    }
    auto mval = [&](uint32_t raw) {
        return EB == 4 ? __uint_as_float(raw) : Elem<T>::widen(raw);
    };

    PointRecord<T, (KT > 0 ? KT * KT : 1)> rec;
    if constexpr (KT > 0) load_record<T, KT * KT>(rec, roff, voff, rmk, vmk, odd);
    __builtin_amdgcn_s_waitcnt(0);     // region, upstream gradient and record have landed
    __syncthreads();
    const char* lds = (const char*)region;

    // one point: returns gm, and writes grad_offset; far corners go to grad_input
    auto point = [&](int q, float2 d, float m) -> float {
        const GradPoint pt = tiled_fetch_grad(G, L, lds, rin, tg.tap_x[q], tg.tap_y[q], d);
        float sk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if constexpr (EB == 4) {
                    acc = fmaf(go[c], __uint_as_float(pt.raw[k][c]), acc);
                } else {
                    acc = fmaf(go[2 * c], Elem<T>::widen(pt.raw[k][c] & 0xffffu), acc);
                    acc = fmaf(go[2 * c + 1], Elem<T>::widen(pt.raw[k][c] >> 16), acc);
                }
            }
            sk[k] = acc;
        }
        const float hy = 1.0f - pt.ly, hx = 1.0f - pt.lx;
        const float wb[4] = {hy * hx, hy * pt.lx, pt.ly * hx, pt.ly * pt.lx};
        float gm = wb[0] * sk[0] + wb[1] * sk[1] + wb[2] * sk[2] + wb[3] * sk[3];
        float gdx = hy * (sk[1] - sk[0]) + pt.ly * (sk[3] - sk[2]);
        float gdy = hx * (sk[2] - sk[0]) + pt.lx * (sk[3] - sk[1]);
        if (tg.gshift >= 1) {
            gm = quad_xor1(gm);
            gdx = quad_xor1(gdx);
            gdy = quad_xor1(gdy);
        }
        if (tg.gshift >= 2) {
            gm = quad_xor2(gm);
            gdx = quad_xor2(gdx);
            gdy = quad_xor2(gdy);
        }
        if (!pt.inmap) { gm = 0.f; gdx = 0.f; gdy = 0.f; }
        if (active && leader) {
            const float gd[2] = {G.alpha * m * gdx, G.alpha * m * gdy};
            store_pair<T>(goff + 2 * q, gd[0], gd[1]);
        }
        // corners beyond the owners' reach: x0 and x0 + 1 both lie within
        // M of the base exactly when x0 - base + M is in [0, 2M) (likewise
        // y), which one test per axis settles for all four corners
        // (unsigned arithmetic: off-map samples carry saturated floors and
        // are excluded below)
        const uint32_t nm = (uint32_t)a.near_m;
        const bool all_near = a.near_m >= 0 && (uint32_t)pt.x0 - (uint32_t)bxi + nm < M2 &&
                              (uint32_t)pt.y0 - (uint32_t)byi + nm < M2;
        if (active && pt.inmap && !all_near) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int qx = pt.x0 + (k & 1), qy = pt.y0 + (k >> 1);
                const bool valid = (uint32_t)qx < (uint32_t)G.W && (uint32_t)qy < (uint32_t)G.H;
                const bool near = a.near_m >= 0 && (uint32_t)(qx - bxi + a.near_m) <= M2 &&
                                  (uint32_t)(qy - byi + a.near_m) <= M2;
                if (valid && !near) {
                    const float mw = m * wb[k];
                    char* px0 = gin + (size_t)qy * G.in_line_bytes + (size_t)qx * G.in_row_bytes;
                    if constexpr (EB == 4) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) atomicAdd((float*)(px0 + L.gl_first) + c, mw * go[c]);
#pragma unroll
                        for (int c = 0; c < 4; ++c) atomicAdd((float*)(px0 + L.gl_second) + c, mw * go[4 + c]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            atomic_add_pair<T>(px0 + L.gl_first + 4 * c, mw * go[2 * c], mw * go[2 * c + 1]);
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            atomic_add_pair<T>(px0 + L.gl_second + 4 * c, mw * go[8 + 2 * c], mw * go[9 + 2 * c]);
                    }
                }
            }
        }
        return gm;
    };

    if constexpr (KT > 0) {
        constexpr int PK = KT * KT;
        float mx = 0.f, inv = 1.f;
        if constexpr (SOFTMAX) {
            mx = mval(rec.mask[0]);
#pragma unroll
            for (int q = 1; q < PK; ++q) mx = fmaxf(mx, mval(rec.mask[q]));
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < PK; ++q) sum += __expf(mval(rec.mask[q]) - mx);
            inv = 1.0f / sum;
        }
        float gms[PK];
        float dot = 0.f;
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            float m = mval(rec.mask[q]);
            if constexpr (SOFTMAX) m = __expf(m - mx) * inv;
            gms[q] = point(q, record_pair<T, PK>(rec, q), m);
            dot = fmaf(m, gms[q], dot);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (active && leader) {
#pragma unroll
            for (int q = 0; q < PK; ++q) {
                float v = gms[q];
                if constexpr (SOFTMAX) v = __expf(mval(rec.mask[q]) - mx) * inv * (v - dot);
                store<T, EB>(gmk + q, &v);
            }
        }
    } else {
        // runtime K: the mask gradients wait in a binary32 array (private
        // memory: the index is not known at compile time) for the softmax
        // Jacobian's dot product
        float mx = 0.f, inv = 1.f;
        if constexpr (SOFTMAX) {
            mx = load_mask_value<T>(rmk, vmk, 0);
            for (int q = 1; q < P; ++q) mx = fmaxf(mx, load_mask_value<T>(rmk, vmk, q));
            float sum = 0.f;
            for (int q = 0; q < P; ++q) sum += __expf(load_mask_value<T>(rmk, vmk, q) - mx);
            inv = 1.0f / sum;
        }
        float gms[kMaxTiledTaps];
        float dot = 0.f;
        for (int q = 0; q < P; ++q) {
            float m = load_mask_value<T>(rmk, vmk, q);
            if constexpr (SOFTMAX) m = __expf(m - mx) * inv;
            gms[q] = point(q, load_offset_pair<T>(roff, voff, q), m);
            dot = fmaf(m, gms[q], dot);
        }
        if (active && leader) {
            for (int q = 0; q < P; ++q) {
                float v = gms[q];
                if constexpr (SOFTMAX) v = __expf(load_mask_value<T>(rmk, vmk, q) - mx) * inv * (v - dot);
                store<T, EB>(gmk + q, &v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// grad_input by owner.  A workgroup owns a TH x TW tile of input pixels and
// one slab of 32 of their channels (four lanes of eight channels per pixel).
// A corner q of a sample of output pixel o is "near" when |q - b(o)| <= M on
// both axes, b(o) = o*stride - pad + c0 being the sample's integer base.  The
// owner visits exactly the output pixels whose base lies within M of its
// tile, recomputes their samples, adds m*w*g of every near corner that falls
// in its tile into an LDS copy of the tile (binary32), and writes the tile
// once, rounded to the dtype.  Each near (sample, corner) pair lies in one
// tile, so grad_input needs neither a zero fill nor global atomics; the rare
// corners that are not near (offsets beyond the reach M was sized for) are
// added afterwards, with atomics, by the gradient kernel.
//
// LDS keeps the tile pixel by pixel, 32 floats each in channel order, at a
// stride of 34 floats: the pixels a wave's lanes add into then start on
// different banks, and a lane's eight channels sit at fixed offsets from one
// 8-byte aligned address.  Lane chunk `sub` adds into floats [8*sub, 8*sub + 8)
// of a pixel.

// Float adds into LDS through compare-and-swap.  On gfx950 an LDS float
// atomic add (ds_add_f32) retires about one lane every few cycles per CU,
// while integer LDS atomics run at the rate of plain LDS accesses; a CAS loop
// uses the latter, on 64-bit words holding two floats each.  The eight adds
// of one lane (consecutive floats) go out together as four swaps of
// old + v; a lane whose swap found another value (another lane added in
// between) repeats the round for its unfinished words, and finished words
// then swap a value for itself, which never changes memory.  Each failed
// swap follows some lane's successful one, so the loop ends.
__device__ __forceinline__ uint64_t add_pair(uint64_t w, float a, float b)
{
    const uint32_t lo = __float_as_uint(__uint_as_float((uint32_t)w) + a);
    const uint32_t hi = __float_as_uint(__uint_as_float((uint32_t)(w >> 32)) + b);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void lds_add8(uint64_t* p, const float (&v)[8])
{
    uint64_t cur[4], des[4], got[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = __hip_atomic_load(p + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        des[j] = add_pair(cur[j], v[2 * j], v[2 * j + 1]);
        got[j] = cur[j];
        __hip_atomic_compare_exchange_strong(p + j, &got[j], des[j], __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    uint32_t pend = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) pend |= (got[j] != cur[j] ? 1u : 0u) << j;
    while (pend) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool retry = (pend >> j) & 1u;
            cur[j] = retry ? got[j] : des[j];
            des[j] = retry ? add_pair(got[j], v[2 * j], v[2 * j + 1]) : des[j];
            got[j] = cur[j];
            __hip_atomic_compare_exchange_strong(p + j, &got[j], des[j], __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        uint32_t again = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) again |= (((pend >> j) & 1u) && got[j] != cur[j] ? 1u : 0u) << j;
        pend = again;
    }
}

constexpr int kOwnerStride = 34;   // floats per pixel in the LDS tile (even: 8-byte words)

struct OwnerGeo {
    int TH, TW, M, Cg;
    uint32_t tiles_x, tiles_y, slabs;
    uint32_t off_image_bytes, mask_image_bytes;   // one image of offset / mask
};

// Output indices o in [0, limit) whose base o*stride - pad + c0 lies in
// [q0 - M, q0 + len - 1 + M].
__device__ __forceinline__ void owner_range(const Geometry& G, int M, int q0, int len, int limit, int& lo, int& hi)
{
    const int a0 = q0 - M + G.pad - G.c0, a1 = q0 + len - 1 + M + G.pad - G.c0;
    lo = a0 <= 0 ? 0 : (a0 + G.stride - 1) / G.stride;
    hi = a1 < 0 ? -1 : a1 / G.stride;
    hi = hi < limit - 1 ? hi : limit - 1;
}

template <typename T, int KT, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4)))
void dcn_backward_input_owner(BwdArgs a, OwnerGeo og)
{
    constexpr int EB = Elem<T>::bytes;
    extern __shared__ float owner_tile[];
    const Geometry& G = a.geo;
    const int t = threadIdx.x;
    uint32_t rest = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t tx = rest % og.tiles_x;
    rest /= og.tiles_x;
    const uint32_t ty = rest % og.tiles_y;
    rest /= og.tiles_y;
    const uint32_t slab = rest % og.slabs;
    const uint32_t n = rest / og.slabs;
    const int qx0 = (int)tx * og.TW, qy0 = (int)ty * og.TH;
    const int tw = og.TW < G.W - qx0 ? og.TW : G.W - qx0;     // ragged last column / row of tiles
    const int th = og.TH < G.H - qy0 ? og.TH : G.H - qy0;

    for (int i = t; i < og.TH * og.TW * kOwnerStride; i += NT) owner_tile[i] = 0.f;
    __syncthreads();

    int wlo, whi, hlo, hhi;
    owner_range(G, og.M, qx0, tw, G.Wo, wlo, whi);
    owner_range(G, og.M, qy0, th, G.Ho, hlo, hhi);
    const int EW = whi - wlo + 1;
    const int E = (EW > 0 && hhi >= hlo) ? EW * (hhi - hlo + 1) : 0;

    const int sub = t & 3;
    const int ch0 = (int)slab * 32 + sub * 8;
    const int g = ch0 / og.Cg;
    const int K = KT > 0 ? KT : G.K;
    const uint32_t M2 = 2u * (uint32_t)og.M;
    const RecordRsrc ro = record_rsrc((const char*)a.offset + (size_t)n * og.off_image_bytes, og.off_image_bytes);
    const __amdgpu_buffer_rsrc_t roff = ro.r;
    const bool odd = EB == 2 && (G.off_stride & 1);   // records on 2-byte boundaries
    const RecordRsrc rm = record_rsrc((const char*)a.mask + (size_t)n * og.mask_image_bytes, og.mask_image_bytes);
    const __amdgpu_buffer_rsrc_t rmk = rm.r;

    // one sample point of output pixel (ho, wo): m*w*g of each near corner in the tile
    auto point = [&](int i, int j, int bxi, int byi, float2 d, float m, const float* go) {
        // the coordinates, skip rule and floor of make_sample
        const float x = fmaf(G.alpha, d.x, fmaf(G.alpha, (float)(i * G.dil - G.c0), (float)bxi));
        const float y = fmaf(G.alpha, d.y, fmaf(G.alpha, (float)(j * G.dil - G.c0), (float)byi));
        if (!(x > -1.0f && x < (float)G.W && y > -1.0f && y < (float)G.H)) return;
        const float fx = floorf(x), fy = floorf(y);
        const int x0 = (int)fx, y0 = (int)fy;
        const int rx = x0 - qx0, ry = y0 - qy0;
        if (rx < -1 || rx >= tw || ry < -1 || ry >= th) return;   // no corner in the tile
        const float lx = x - fx, ly = y - fy;
        const float hy = 1.0f - ly, hx = 1.0f - lx;
        const float wb[4] = {hy * hx, hy * lx, ly * hx, ly * lx};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int cx = rx + (k & 1), cy = ry + (k >> 1);
            const int qx = x0 + (k & 1), qy = y0 + (k >> 1);
            const bool mine = (uint32_t)cx < (uint32_t)tw && (uint32_t)cy < (uint32_t)th &&
                              (uint32_t)(qx - bxi + og.M) <= M2 && (uint32_t)(qy - byi + og.M) <= M2;
            if (mine) {
                const float mw = m * wb[k];
                // 24-bit multiply: a 64-bit multiply-add here reads a register
                // pair whose upper half may be a load still in flight
                const uint32_t base = (__umul24((uint32_t)cy, (uint32_t)og.TW) + (uint32_t)cx) * (uint32_t)kOwnerStride +
                                      (uint32_t)sub * 8u;
                float v[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) v[c] = mw * go[c];
                lds_add8((uint64_t*)(owner_tile + base), v);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Each lane walks the visited output pixels in steps of NT/4, fetching a
    // pixel's upstream gradient and whole records at once.  (Holding
    // the next pixel's fetch in registers as well spills at this register
    // budget and measured slower.)
    struct Pending {
        uint32_t gw[2 * EB];                  // the lane's 8 upstream-gradient elements
        PointRecord<T, (KT > 0 ? KT * KT : 1)> rec;
    };
    auto fetch = [&](int ho, int wo, Pending& pd) {
        const size_t pix = ((size_t)n * G.Ho + ho) * G.Wo + wo;
        const uint4* gp = (const uint4*)((const char*)a.grad_out + (pix * G.C + ch0) * EB);
#pragma unroll
        for (int h = 0; h < EB / 2; ++h) {
            const uint4 v = gp[h];
            pd.gw[4 * h] = v.x; pd.gw[4 * h + 1] = v.y; pd.gw[4 * h + 2] = v.z; pd.gw[4 * h + 3] = v.w;
        }
        if constexpr (KT > 0) {
            const uint32_t pg_img = ((uint32_t)ho * (uint32_t)G.Wo + (uint32_t)wo) * (uint32_t)G.groups + (uint32_t)g;
            load_record<T, KT * KT>(pd.rec, roff, pg_img * (uint32_t)(G.off_stride * EB) + ro.lead, rmk,
                                    pg_img * (uint32_t)(G.mask_stride * EB) + rm.lead, odd);
        }
    };
    auto mval = [&](uint32_t raw) {
        return EB == 4 ? __uint_as_float(raw) : Elem<T>::widen(raw);
    };

    // Visit order: the rows of the visited window split into four phases
    // (row mod 4); within a phase, column by column.  A wave's 16 pixel
    // slots are consecutive in this order, so they share a column: the
    // window's margin columns, whose samples rarely reach the tile, fill
    // waves of their own that skip most corners together (mixing them into
    // every wave cost 16% more time on the 56x56 fp32 stage).  The slots sit
    // 4 rows apart, so two lanes of one LDS instruction rarely add into one
    // address.
    const int EH = E > 0 ? E / EW : 0;
    int cum[5];
    cum[0] = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) cum[p + 1] = cum[p] + EW * ((EH - p + 3) >> 2);
    const int e0 = t >> 2;
    for (int e = e0; e < E; e += NT / 4) {
        const int ph = (e >= cum[1]) + (e >= cum[2]) + (e >= cum[3]);   // cum[ph] <= e < cum[ph + 1]
        const int cnt = (EH - ph + 3) >> 2, local = e - cum[ph];
        const int col = local / cnt, k = local - col * cnt;
        const int ho = hlo + ph + 4 * k, wo = wlo + col;
        Pending cur;
        fetch(ho, wo, cur);
        const int bxi = wo * G.stride - G.pad + G.c0, byi = ho * G.stride - G.pad + G.c0;
        float go[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (EB == 4) go[c] = __uint_as_float(cur.gw[c]);
            else go[c] = Elem<T>::widen((c & 1) ? cur.gw[c >> 1] >> 16 : cur.gw[c >> 1] & 0xffffu);
        }
        if constexpr (KT > 0) {
            constexpr int PK = KT * KT;
            float mx = 0.f, inv = 1.f;
            if (G.softmax) {
                mx = mval(cur.rec.mask[0]);
#pragma unroll
                for (int q = 1; q < PK; ++q) mx = fmaxf(mx, mval(cur.rec.mask[q]));
                float sum = 0.f;
#pragma unroll
                for (int q = 0; q < PK; ++q) sum += __expf(mval(cur.rec.mask[q]) - mx);
                inv = 1.0f / sum;
            }
#pragma unroll
            for (int i = 0; i < KT; ++i)
#pragma unroll
                for (int j = 0; j < KT; ++j) {
                    const int q = i * KT + j;
                    float m = mval(cur.rec.mask[q]);
                    if (G.softmax) m = __expf(m - mx) * inv;
                    point(i, j, bxi, byi, record_pair<T, PK>(cur.rec, q), m, go);
                }
        } else {
            const size_t pg = (((size_t)n * G.Ho + ho) * G.Wo + wo) * G.groups + g;
            const T* off = (const T*)a.offset + pg * G.off_stride;
            const T* mk = (const T*)a.mask + pg * G.mask_stride;
            float mx = 0.f, inv = 1.f;
            if (G.softmax) {
                mx = ld1(mk);
                for (int q = 1; q < G.P; ++q) mx = fmaxf(mx, ld1(mk + q));
                float sum = 0.f;
                for (int q = 0; q < G.P; ++q) sum += __expf(ld1(mk + q) - mx);
                inv = 1.0f / sum;
            }
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < K; ++j) {
                    const int q = point_of(G, i, j);
                    if (q < 0) continue;
                    float m = ld1(mk + q);
                    if (G.softmax) m = __expf(m - mx) * inv;
                    point(i, j, bxi, byi, ld2(off + 2 * q), m, go);
                }
        }
    }
    __syncthreads();

    // write the tile, 4 channels per lane, rounded once to the dtype
    char* gin = (char*)a.grad_input + (size_t)n * G.in_image_bytes + slab * (32u * EB);
    for (int i = t; i < th * tw * 8; i += NT) {
        const int px = i >> 3, q4 = i & 7;
        const int cy = px / tw, cx = px - cy * tw;
        const int qx = qx0 + cx, qy = qy0 + cy;
        const float* src = owner_tile + (cy * og.TW + cx) * kOwnerStride + q4 * 4;
        const float v[4] = {src[0], src[1], src[2], src[3]};
        store<T, 4 * EB>(gin + (size_t)qy * G.in_line_bytes + (size_t)qx * G.in_row_bytes + q4 * (4 * EB), v);
    }
}

// ---------------------------------------------------------------------------
// Half-precision backward for the shapes the tiled kernels do not take: the
// lane mapping and arithmetic of dcn_backward_kernel (the binary32 fallback)
// on half-precision tensors, with every grad_input contribution added by a
// binary32 atomic into a caller's workspace (N*H*W*C floats, zeroed first)
// that dcn_store_workspace then rounds once into grad_input.  L, the lanes of
// one group (a power of two up to 64), is a runtime value here.
__device__ __forceinline__ float group_sum_rt(float v, int L)
{
    for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <typename T, int LB, int KT>
__global__ __launch_bounds__(kBlock) void dcn_backward_generic(BwdArgs a, float* ws, int L)
{
    constexpr int EB = Elem<T>::bytes;
    constexpr int CPL = LB / EB;
    const Geometry& G = a.geo;
    const LaneWork lw = lane_work(G);
    // inactive lanes (past the image) stay for the cross-lane sums but touch
    // no memory; a group is always wholly active or wholly inactive
    const bool act = lw.active;

    const char* in_img = (const char*)a.input + (size_t)lw.n * G.in_image_bytes;
    const __amdgpu_buffer_rsrc_t rin = image_rsrc(in_img, G.in_image_bytes);
    const uint32_t chan_bytes = lw.cc * (CPL * EB);
    const size_t pix_global = (size_t)lw.n * G.Ho * G.Wo + lw.pix;
    const size_t pg = pix_global * G.groups + lw.g;
    const T* off = (const T*)a.offset + pg * G.off_stride;
    const T* mk = (const T*)a.mask + pg * G.mask_stride;
    T* goff = (T*)a.grad_offset + pg * G.off_stride;
    T* gmk = (T*)a.grad_mask + pg * G.mask_stride;
    float* wimg = ws + (size_t)lw.n * (G.in_image_bytes / EB);
    const int bxi = (int)lw.wo * G.stride - G.pad + G.c0;
    const int byi = (int)lw.ho * G.stride - G.pad + G.c0;
    const float bx = (float)bxi, by = (float)byi;
    const bool leader = (lw.cc & (uint32_t)(L - 1)) == 0;

    float go[CPL];
    {
        const T* gp = (const T*)a.grad_out + pix_global * G.C + lw.cc * CPL;
#pragma unroll
        for (int c = 0; c < CPL; ++c) go[c] = act ? ld1(gp + c) : 0.f;
    }
    float mx = 0.f, inv = 1.f;
    if (G.softmax && act) {
        mx = ld1(mk);
        for (int p = 1; p < G.P; ++p) mx = fmaxf(mx, ld1(mk + p));
        float sum = 0.f;
        for (int p = 0; p < G.P; ++p) sum += __expf(ld1(mk + p) - mx);
        inv = 1.0f / sum;
    }
    float dot = 0.f;   // sum_q m_q gm_q (softmax)

    const int K = KT > 0 ? KT : G.K;
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < K; ++j) {
            const int p = point_of(G, i, j);
            if (p < 0) continue;                                // (the same for every lane)
            float m = 0.f;
            float2 d = make_float2(__builtin_nanf(""), 0.f);   // inactive: never on the map
            if (act) {
                m = ld1(mk + p);
                if (G.softmax) m = __expf(m - mx) * inv;
                d = ld2(off + 2 * p);
            }
            const Sample s = make_sample(G, bx, by, i, j, d.x, d.y, chan_bytes);
            const float hy = 1.0f - s.ly, hx = 1.0f - s.lx;
            const float wb[4] = {hy * hx, hy * s.lx, s.ly * hx, s.ly * s.lx};
            const float dwx[4] = {-hy, hy, -s.ly, s.ly};
            const float dwy[4] = {-hx, -s.lx, hx, s.lx};
            float gm = 0.f, gdx = 0.f, gdy = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float f[CPL];
                gather<T, LB>(rin, s.off[k], f);
                float sk = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) sk = fmaf(go[c], f[c], sk);
                gm = fmaf(wb[k], sk, gm);
                gdx = fmaf(dwx[k], sk, gdx);
                gdy = fmaf(dwy[k], sk, gdy);
                if (s.v[k]) {
                    const float mw = m * wb[k];
                    float* dst = wimg + s.off[k] / EB;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) atomicAdd(dst + c, mw * go[c]);
                }
            }
            gm = group_sum_rt(gm, L);
            gdx = group_sum_rt(gdx, L);
            gdy = group_sum_rt(gdy, L);
            if (!s.inmap) { gm = 0.f; gdx = 0.f; gdy = 0.f; }
            if (act && leader) {
                store_pair<T>(goff + 2 * p, G.alpha * m * gdx, G.alpha * m * gdy);
                store<T, EB>(gmk + p, &gm);
            }
            dot = fmaf(m, gm, dot);
        }
    if (G.softmax && act && leader) {
        // second pass over the stored raw gm (rounded once to the dtype)
        for (int p = 0; p < G.P; ++p) {
            const float m = __expf(ld1(mk + p) - mx) * inv;
            const float v = m * (ld1(gmk + p) - dot);
            store<T, EB>(gmk + p, &v);
        }
    }
}

// grad_input = the binary32 workspace, rounded once to the dtype
template <typename T>
__global__ __launch_bounds__(kBlock) void dcn_store_workspace(const float* ws, T* gi, size_t n)
{
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) store<T, Elem<T>::bytes>(gi + i, ws + i);
}

// Zero fill on the caller's stream (a kernel rather than a memset node, so
// a caller may capture the call in a graph).
__global__ __launch_bounds__(kBlock) void dcn_zero_kernel(float4* p, size_t n4, float* tail, int ntail)
{
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0.f;
}

}  // namespace dcn
