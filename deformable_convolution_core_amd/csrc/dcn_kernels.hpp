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

// mixed_fma: the mixed-precision FMA (v_fma_mix_f32) reads the type's values
// directly, with no separate widening instruction.
template <> struct Elem<float> {
    static constexpr int bytes = 4;
    static constexpr bool mixed_fma = false;
    __device__ static float widen(uint32_t u) { return __uint_as_float(u); }
    __device__ static uint32_t narrow(float f) { return __float_as_uint(f); }
};
template <> struct Elem<_Float16> {
    static constexpr int bytes = 2;
    static constexpr bool mixed_fma = true;
    __device__ static float widen(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)u); }
    // The value is pinned first: the compiler may otherwise fuse the last
    // binary32 fma of a sum with this conversion (v_fma_mixlo_f16, one
    // rounding straight to fp16), which is not "a binary32 sum rounded once".
    __device__ static uint32_t narrow(float f)
    {
        asm volatile("" : "+v"(f));
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
};
template <> struct Elem<__bf16> {
    static constexpr int bytes = 2;
    static constexpr bool mixed_fma = false;
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
    // Half precision: the gradient kernel adds the corners that are not near
    // into this binary32 image of grad_input (zeroed first), and the owner
    // kernel starts its tiles from it (gi_init), so every grad_input element
    // is a binary32 sum rounded once.  Null for binary32 calls.
    float* far_ws;
    const float* gi_init;
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

// Per-lane constants of the tiled kernel's compute phase.  The point loop
// reads the uniform ones from VGPR copies (vgpr_copy): on gfx950 a VALU
// instruction with an SGPR operand issues at about 0.6x the rate of the same
// instruction with VGPR operands only.
struct TiledLane {
    float bx, by;                 // sampling centre (absolute input coordinates)
    int x_lo, y_lo;               // staged region origin
    uint32_t xlim, ylim;          // RW-1, RH-1 (the gradient kernel's region test)
    uint32_t lane_first;          // this lane's first 16-byte slot in a pixel slab
    uint32_t RW, RWB;             // region width in pixels and in bytes
    uint32_t gl_first, gl_second; // the two halves inside an input pixel row
    // Fast-path bounds: lox < x < hix and loy < y < hiy hold exactly when the
    // sample is on the map (x > -1, x < W, likewise y) and its four corners
    // lie in the staged region (x_lo <= floor(x) <= x_lo + RW - 2).  A NaN
    // coordinate fails them.
    float lox, hix, loy, hiy;
    float w_f, h_f;               // W, H
    float alpha;
    float rwb_f, addr_base;       // LDS address of pixel (fy, fx) = fy*rwb_f + fx*128 + addr_base
    uint32_t zero_a0;             // this lane's slot in a 2x2 block of zero pixels
};

// A uniform value copied into a VGPR the compiler cannot see through.
__device__ __forceinline__ float vgpr_copy(float s)
{
    float v;
    asm volatile("" : "=v"(v) : "0"(s));
    return v;
}
__device__ __forceinline__ uint32_t vgpr_copy(uint32_t s)
{
    uint32_t v;
    asm volatile("" : "=v"(v) : "0"(s));
    return v;
}

// v_cvt_u32_f32: in-range non-negative integers convert exactly; anything
// else (NaN, negative, huge) gives some value the caller then discards.
__device__ __forceinline__ uint32_t cvt_u32(float x)
{
    uint32_t r;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Strict lower bound equivalent to "x >= lo and x > -1" for an integer lo:
// the float just below lo (lo >= 1), -1 (lo <= -1).  For lo = 0 the bound is
// -0.0, which also turns away x = 0 itself; such a sample takes the slower
// path, which gives the same result.
__device__ __forceinline__ float fast_lower_bound(int lo)
{
    return lo >= 1 ? __int_as_float(__float_as_int((float)lo) - 1) : (lo == 0 ? -0.0f : -1.0f);
}

// whole: the region is the whole map with a one-pixel zero border (origin
// -1, -1) and two zero rows below it, so every sample on the map is inside
// it and the zero block is rows H + 1, H + 2 of the region; otherwise the
// zero block follows the region's RH rows.
__device__ __forceinline__ void set_fast_bounds(TiledLane& L, const Geometry& G, uint32_t RH, bool whole)
{
    if (whole) {
        L.lox = -1.0f;
        L.loy = -1.0f;
        L.hix = (float)G.W;
        L.hiy = (float)G.H;
        L.zero_a0 = (uint32_t)(G.H + 1) * L.RWB + L.lane_first;
    } else {
        L.lox = fast_lower_bound(L.x_lo);
        L.loy = fast_lower_bound(L.y_lo);
        const int hx = L.x_lo + (int)L.RW - 1, hy = L.y_lo + (int)RH - 1;
        L.hix = (float)(hx < G.W ? hx : G.W);
        L.hiy = (float)(hy < G.H ? hy : G.H);
        L.zero_a0 = RH * L.RWB + L.lane_first;
    }
    L.lox = vgpr_copy(L.lox);
    L.loy = vgpr_copy(L.loy);
    L.hix = vgpr_copy(L.hix);
    L.hiy = vgpr_copy(L.hiy);
    L.zero_a0 = vgpr_copy(L.zero_a0);
    L.w_f = vgpr_copy((float)G.W);
    L.h_f = vgpr_copy((float)G.H);
    L.alpha = vgpr_copy(G.alpha);
    L.rwb_f = vgpr_copy((float)L.RWB);
    L.addr_base = (float)L.lane_first - (float)L.y_lo * (float)L.RWB - (float)L.x_lo * 128.0f;
}

// Bilinear weights with the modulation folded in; each is formed with
// relative error <= 2 ulp (the one-minus factors are fused, so a weight near
// zero is not the difference of two rounded values).
__device__ __forceinline__ void modulated_weights(float mm, float lx, float ly, float* w)
{
    const float mly = mm * ly, mhy = fmaf(-mm, ly, mm);
    w[0] = fmaf(-mhy, lx, mhy);
    w[1] = mhy * lx;
    w[2] = fmaf(-mly, lx, mly);
    w[3] = mly * lx;
}

template <typename T>
__device__ __forceinline__ void accumulate_corner(const uint32_t (&raw)[8], float w, float* acc)
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        if constexpr (Elem<T>::bytes == 4) {
            acc[c] = fmaf(w, __uint_as_float(raw[c]), acc[c]);
        } else {
            acc[2 * c] = fmaf(w, Elem<T>::widen(raw[c] & 0xffffu), acc[2 * c]);
            acc[2 * c + 1] = fmaf(w, Elem<T>::widen(raw[c] >> 16), acc[2 * c + 1]);
        }
    }
}

// Coordinates, weights and corner reads of one point from the staged region.
// A sample that the region does not serve -- off the map (the definition
// skips it), NaN, or on the map beyond the region -- reads the block of
// zeros with zero weights instead, so an Inf or NaN in the input can never
// meet a zero weight here; far is set for the last kind (never in a
// whole-map region), whose corners the caller gathers from memory
// (far_accumulate).  xt, yt: the tap's part of the coordinates,
// fmaf(alpha, tap, base).  Floor and fraction come from the absolute
// coordinate; the LDS address is formed in binary32 from the floors, exactly
// (every term is an integer below 2^24).
template <typename T, bool WHOLE>
__device__ __forceinline__ TiledPoint tiled_fetch(const TiledLane& L, const char* lds, float xt, float yt, float2 d,
                                                  float m, bool& far, float& x, float& y)
{
    TiledPoint pt;
    x = fmaf(L.alpha, d.x, xt);
    y = fmaf(L.alpha, d.y, yt);
    const float fx = floorf(x), fy = floorf(y);
    const bool ok = (x > L.lox) & (x < L.hix) & (y > L.loy) & (y < L.hiy);
    float lx = x - fx, ly = y - fy, mm = m;
    uint32_t a0 = cvt_u32(fmaf(fy, L.rwb_f, fmaf(fx, 128.0f, L.addr_base)));
    far = false;
    if (!ok) {
        a0 = L.zero_a0;
        lx = 0.f;
        ly = 0.f;
        mm = 0.f;
        if constexpr (!WHOLE) far = (x > -1.0f) & (x < L.w_f) & (y > -1.0f) & (y < L.h_f);
    }
    const uint32_t a1 = a0 ^ 16u;
    const uint32_t b0 = a0 + L.RWB, b1 = a1 + L.RWB;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t p0 = k ? b0 : a0, p1 = k ? b1 : a1;
        const uint4 v00 = *(const uint4*)(lds + p0);
        const uint4 v01 = *(const uint4*)(lds + p1);
        const uint4 v10 = *(const uint4*)(lds + p0 + 128u);
        const uint4 v11 = *(const uint4*)(lds + p1 + 128u);
        uint32_t* r0 = pt.raw[2 * k];
        uint32_t* r1 = pt.raw[2 * k + 1];
        r0[0] = v00.x; r0[1] = v00.y; r0[2] = v00.z; r0[3] = v00.w;
        r0[4] = v01.x; r0[5] = v01.y; r0[6] = v01.z; r0[7] = v01.w;
        r1[0] = v10.x; r1[1] = v10.y; r1[2] = v10.z; r1[3] = v10.w;
        r1[4] = v11.x; r1[5] = v11.y; r1[6] = v11.z; r1[7] = v11.w;
    }
    modulated_weights(mm, lx, ly, pt.w);
    return pt;
}

// A sample on the map whose corners fall outside the staged region: gather
// its four corner rows from memory (off-map corners read zeros through the
// buffer resource) and accumulate them.  Self-contained, so the loads' wait
// stays inside this rarely taken branch.
template <typename T>
__device__ __forceinline__ void far_accumulate(const Geometry& G, const TiledLane& L, __amdgpu_buffer_rsrc_t rin,
                                               float x, float y, float m, float* acc)
{
    const float fx = floorf(x), fy = floorf(y);
    float w[4];
    modulated_weights(m, x - fx, y - fy, w);
    const int x0 = (int)fx, y0 = (int)fy;
    const bool vx0 = (uint32_t)x0 < (uint32_t)G.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)G.W;
    const bool vy0 = (uint32_t)y0 < (uint32_t)G.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)G.H;
    const bool vk[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
    const uint32_t a00 = (uint32_t)y0 * G.in_line_bytes + (uint32_t)x0 * G.in_row_bytes;
    const uint32_t ck[4] = {0u, G.in_row_bytes, G.in_line_bytes, G.in_line_bytes + G.in_row_bytes};
    uint32_t raw[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t o0 = vk[k] ? a00 + ck[k] + L.gl_first : kOOB;
        const uint32_t o1 = vk[k] ? a00 + ck[k] + L.gl_second : kOOB;
        const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rin, o0, 0, 0);
        const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rin, o1, 0, 0);
        raw[k][0] = v0[0]; raw[k][1] = v0[1]; raw[k][2] = v0[2]; raw[k][3] = v0[3];
        raw[k][4] = v1[0]; raw[k][5] = v1[1]; raw[k][6] = v1[2]; raw[k][7] = v1[3];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) accumulate_corner<T>(raw[k], w[k], acc);
}

// Ordering point between two sampling points: the accumulators pass through
// it (so this point's fmas come first) and it clobbers memory (so the next
// point's LDS reads come after).  Without it the compiler issues every
// point's corner reads up front and spills the rows it cannot hold.
template <int CPL>
__device__ __forceinline__ void point_fence(float* acc)
{
    if constexpr (CPL == 16) {
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                     "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]), "+v"(acc[9]), "+v"(acc[10]), "+v"(acc[11]),
                     "+v"(acc[12]), "+v"(acc[13]), "+v"(acc[14]), "+v"(acc[15])::"memory");
    } else {
        static_assert(CPL == 8, "channels per lane");
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                     "+v"(acc[6]), "+v"(acc[7])::"memory");
    }
}

template <typename T, int CPL>
__device__ __forceinline__ void tiled_accumulate(const TiledPoint& pt, float* acc)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) accumulate_corner<T>(pt.raw[k], pt.w[k], acc);
}

// Image, slab and region origin of one tile (wave-uniform values).
struct TileCoord {
    uint32_t n, slab;
    int ho0, wo0, y_lo, x_lo;
};

__device__ __forceinline__ TileCoord tile_coord(const Geometry& G, const TileGeo& tg, uint32_t tile)
{
    TileCoord c;
    // the slab varies fastest: the slabs of one tile run as neighbouring
    // tiles of one XCD, so the cache lines of a pixel's offset and mask
    // records that two slabs' groups share meet in that XCD's L2 (read once,
    // and written back once by the gradient kernel)
    uint32_t rest = tile;
    c.slab = rest % tg.slabs;
    rest /= tg.slabs;
    const uint32_t tx = rest % tg.tiles_x;
    rest /= tg.tiles_x;
    const uint32_t ty = rest % tg.tiles_y;
    c.n = rest / tg.tiles_y;
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
// rows a lane steps its offset by one image row.  NT: the block's lanes, a
// multiple of 64.
__device__ __forceinline__ void stage_rows(const Geometry& G, const TileGeo& tg, const void* input,
                                           const TileCoord& c, uint4* buf, int r0, int r1, int t, int NT)
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

    // The staging and record loads are issued at a raised wave priority, so
    // that a workgroup arriving on a CU gets its memory requests out ahead of
    // the point loop of the workgroup already there; the priority drops back
    // before the wait.  (Measured: 2-5% off the large-shape launches.)
    __builtin_amdgcn_s_setprio(1);
    const TileCoord cur = tile_coord(G, tg, xcd_remap(blockIdx.x, gridDim.x));
    stage_rows(G, tg, a.input, cur, region, 0, tg.RH, t, (int)blockDim.x);
    if constexpr (!WHOLE) {
        // the 2x2 block of zero pixels after the region (rows RH and RH + 1,
        // columns 0 and 1 at the region's row stride): 32 lanes, 16 bytes each
        if (t < 32) {
            const int k = t >> 3;
            region[((tg.RH + (k >> 1)) * tg.RW + (k & 1)) * 8 + (t & 7)] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

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
    set_fast_bounds(L, G, (uint32_t)tg.RH, WHOLE);
    const char* lds = (const char*)region;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    auto acc_ref = [&]() -> float* { return acc; };

    auto mval = [&](uint32_t raw) {
        return Elem<T>::bytes == 4 ? __uint_as_float(raw) : Elem<T>::widen(raw);
    };
    // one point: its corners from the staged region (the whole-map variant
    // needs nothing else), plus the memory gather of a sample on the map
    // beyond the region
    // Lanes past the tile (or the map) run the points too, on a valid record
    // and valid reads, and store nothing: no branch per point.
    auto point = [&](float xt, float yt, float2 d, float m) {
        bool far;
        float x, y;
        tiled_accumulate<T, CPL>(tiled_fetch<T, WHOLE>(L, lds, xt, yt, d, m, far, x, y), acc_ref());
        if constexpr (!WHOLE) {
            if (far) far_accumulate<T>(G, L, rin, x, y, m, acc_ref());
        }
    };
    float zval = 0.f;
    if constexpr (GATE) {
        // the gate logit, in flight with the record and the region
        if (active) zval = ld1((const T*)a.gate + (size_t)cur.n * G.Ho * G.Wo * G.groups + pg_img);
    }
    if constexpr (KT > 0) {
        // K fixed: the (pixel, group)'s offset and mask records come in once
        // (a per-point load would re-touch the same cache lines P times)
        // and the points are unrolled so the record stays in registers.
        constexpr int PK = KT * KT;
        PointRecord<T, PK> rec;
        load_record<T, PK>(rec, roff, voff, rmk, vmk, odd);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(0);   // the region (and the record) have landed
        __syncthreads();
        // the modulation: raw, or the softmax over the PK points (each
        // exponential formed once)
        float mq[PK];
#pragma unroll
        for (int q = 0; q < PK; ++q) mq[q] = mval(rec.mask[q]);
        if constexpr (SOFTMAX) {
            float mx = mq[0];
#pragma unroll
            for (int q = 1; q < PK; ++q) mx = fmaxf(mx, mq[q]);
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < PK; ++q) {
                mq[q] = __expf(mq[q] - mx);
                sum += mq[q];
            }
            const float inv = 1.0f / sum;
#pragma unroll
            for (int q = 0; q < PK; ++q) mq[q] *= inv;
        }
        // the taps' part of the coordinates, once per column and row of taps
        float xt[KT], yt[KT];
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            xt[i] = fmaf(L.alpha, tg.tap_x[i * KT], L.bx);
            yt[i] = fmaf(L.alpha, tg.tap_y[i], L.by);
        }
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            point(xt[q / KT], yt[q % KT], record_pair<T, PK>(rec, q), mq[q]);
            point_fence<CPL>(acc);
        }
    } else {
        __builtin_amdgcn_s_setprio(0);
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
        // one point per (rolled) iteration; its offset pair and mask value
        // are requested one point ahead
        RawPair<T> dn = load_offset_raw<T>(roff, voff, 0, odd);
        uint32_t mn = load_mask_raw<T>(rmk, vmk, 0);
        DCN_UNROLL(1)
        for (int q = 0; q < P; ++q) {
            const RawPair<T> d = dn;
            const uint32_t mraw = mn;
            if (q + 1 < P) { dn = load_offset_raw<T>(roff, voff, q + 1, odd); mn = load_mask_raw<T>(rmk, vmk, q + 1); }
            float m = mval(mraw);
            if constexpr (SOFTMAX) m = __expf(m - mx) * inv;
            point(fmaf(L.alpha, tg.tap_x[q], L.bx), fmaf(L.alpha, tg.tap_y[q], L.by), widen_pair<T>(d), m);
            point_fence<CPL>(acc);
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
            // the owner kernel added the corners of samples whose four
            // corners lie within near_m of the sampling base
            const bool near = a.near_m >= 0 && (uint32_t)(s.x0 - bxi + a.near_m) < 2u * (uint32_t)a.near_m &&
                              (uint32_t)(s.y0 - byi + a.near_m) < 2u * (uint32_t)a.near_m;
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
            // a skipped sample has zero gradients whatever its mask value
            // (an Inf or NaN it never multiplies must not meet the zeros)
            if (!s.inmap) { gm = 0.f; gdx = 0.f; gdy = 0.f; }
            const float am = s.inmap ? G.alpha * m : 0.f;
            if (act && leader) {
                *(float2*)(goff + 2 * p) = make_float2(am * gdx, am * gdy);
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
    stage_rows(G, tg, a.input, cur, region, 0, tg.RH, t, (int)blockDim.x);

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
        // a skipped sample has zero gradients whatever its mask value
        if (!pt.inmap) { gm = 0.f; gdx = 0.f; gdy = 0.f; }
        if (active && leader) {
            const float am = pt.inmap ? G.alpha * m : 0.f;
            store_pair<T>(goff + 2 * q, am * gdx, am * gdy);
        }
        // samples beyond the owners' reach: the owners took the corners of
        // every sample whose x0 and x0 + 1 both lie within M of the base,
        // that is x0 - base + M in [0, 2M) (likewise y); the corners of the
        // others are added here (unsigned arithmetic: off-map samples carry
        // saturated floors and are excluded below)
        const uint32_t nm = (uint32_t)a.near_m;
        const bool near = a.near_m >= 0 && (uint32_t)pt.x0 - (uint32_t)bxi + nm < M2 &&
                          (uint32_t)pt.y0 - (uint32_t)byi + nm < M2;
        if (active && pt.inmap && !near) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int qx = pt.x0 + (k & 1), qy = pt.y0 + (k >> 1);
                const bool valid = (uint32_t)qx < (uint32_t)G.W && (uint32_t)qy < (uint32_t)G.H;
                if (valid) {
                    const float mw = m * wb[k];
                    const size_t pix_el = (size_t)qy * G.W * G.C + (size_t)qx * G.C;   // elements
                    if constexpr (EB == 4) {
                        float* px0 = (float*)gin + pix_el;
#pragma unroll
                        for (int c = 0; c < 4; ++c) atomicAdd(px0 + L.gl_first / 4 + c, mw * go[c]);
#pragma unroll
                        for (int c = 0; c < 4; ++c) atomicAdd(px0 + L.gl_second / 4 + c, mw * go[4 + c]);
                    } else {
                        // binary32 adds into the workspace image of grad_input
                        float* px0 = a.far_ws + (size_t)cur.n * G.H * G.W * G.C + pix_el;
#pragma unroll
                        for (int c = 0; c < 8; ++c) atomicAdd(px0 + L.gl_first / 2 + c, mw * go[c]);
#pragma unroll
                        for (int c = 0; c < 8; ++c) atomicAdd(px0 + L.gl_second / 2 + c, mw * go[8 + c]);
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
        // the softmax Jacobian needs every point's mask gradient first; a raw
        // mask's gradient is stored as soon as it is known
        float gms[SOFTMAX ? PK : 1];
        float dot = 0.f;
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            float m = mval(rec.mask[q]);
            if constexpr (SOFTMAX) m = __expf(m - mx) * inv;
            const float gq = point(q, record_pair<T, PK>(rec, q), m);
            if constexpr (SOFTMAX) {
                gms[q] = gq;
                dot = fmaf(m, gq, dot);
            } else if (active && leader) {
                store<T, EB>(gmk + q, &gq);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SOFTMAX) {
            if (active && leader) {
#pragma unroll
                for (int q = 0; q < PK; ++q) {
                    const float v = __expf(mval(rec.mask[q]) - mx) * inv * (gms[q] - dot);
                    store<T, EB>(gmk + q, &v);
                }
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
// grad_input by owner.  A workgroup owns a TH x TW tile of input pixels of one
// image and one group.  A sample of output pixel o is "near" when its four
// corners lie within M of b(o) = o*stride - pad + c0, the sample's integer
// base, on both axes (x0 - b in [-M, M - 1], likewise y0).  The owner visits
// exactly the output pixels whose base lies within M of its tile, recomputes
// their samples, and sums m*w*g over the corners of near samples that fall in
// its tile, in binary32, each tile element in one lane's registers; it
// writes the tile once, rounded to the dtype.  Each corner of a near sample
// lies in one tile, so grad_input needs neither a zero fill nor global
// atomics; the corners of the rare samples that are not near (offsets beyond
// the reach M was sized for) are added afterwards, with atomics, by the
// gradient kernel.
//
// The sums are gathers, not scatters: the visited output pixels are taken in
// chunks of interleaved rows, and within a chunk every near sample whose 2x2
// neighbourhood touches the tile is sorted by its top-left corner (x0, y0)
// into bins, one per position in [qx0 - 1, qx0 + tw - 1] x
// [qy0 - 1, qy0 + th - 1], with a counting sort: integer LDS atomics count
// the bins, a block scan turns the counts into bin starts, and a second visit
// places each sample's record (where its output pixel's gradient row sits in
// LDS, m, the fractions lx, ly) at the next free slot of its bin.  The pixel
// at tile position (cx, cy) is the (dx, dy) corner of exactly the samples in
// the 2x2 bins (cx + 1 - dx, cy + 1 - dy); those are two runs of consecutive
// records (bins are numbered row by row), which its lane walks, weighting
// each record's upstream-gradient row (staged in LDS, binary32) by m times
// the bilinear weight of that corner.  LDS float atomics, which gfx950
// retires far slower than integer ones, are not used.
//
// While a chunk's records are gathered, every lane already holds the loads
// of the next chunk (its output pixel's offset and mask record and its share
// of the gradient rows), so the global-memory latency of a chunk hides behind
// the previous chunk's gather.  A chunk takes at most one record slot per
// sample (rows * window width * P), which the planner sizes the chunk for, so
// one sort always holds the whole chunk.

// Output indices o in [0, limit) whose base o*stride - pad + c0 lies in
// [q0 - M, q0 + len - 1 + M].
__device__ __forceinline__ void owner_range(const Geometry& G, int M, int q0, int len, int limit, int& lo, int& hi)
{
    const int a0 = q0 - M + G.pad - G.c0, a1 = q0 + len - 1 + M + G.pad - G.c0;
    lo = a0 <= 0 ? 0 : (a0 + G.stride - 1) / G.stride;
    hi = a1 < 0 ? -1 : a1 / G.stride;
    hi = hi < limit - 1 ? hi : limit - 1;
}

constexpr int kBinPrefetch = 4;   // 16-byte gradient pieces a lane holds for the next chunk, at most
constexpr int kBinSamples = 6;    // samples a lane holds for the next chunk, at most

struct BinGeo {
    int TH, TW, M;               // tile of input pixels; reach
    int Cg;                      // channels per group
    int R;                       // visited output rows per chunk
    int ew_max;                  // visited output columns, at most
    int cap;                     // record slots: R * ew_max * P
    int nb_max;                  // bins: (TH + 1) * (TW + 1)
    uint32_t tiles_x, tiles_y;
    uint32_t off_image_bytes, mask_image_bytes;   // one image of offset / mask
    uint32_t gout_image_bytes;                    // one image of grad_output (< 2^31)
    int eb;                                       // bytes per staged gradient element: 2 for fp16, else 4
};

// Bytes per staged gradient row (the group's Cg elements of eb bytes each)
// plus 16, so that rows start on different 16-byte bank groups and
// random rows read together rarely collide.
__host__ __device__ inline int bin_row_bytes(int Cg, int eb) { return Cg * eb + 16; }

// LDS of one workgroup, in this order: bin counts and bin starts (nb_max + 1,
// the last one the total), one total per wave for the scan, the records (16
// bytes each), the staged upstream gradient (rows of eb-byte elements:
// binary32, or fp16 for fp16 calls), a row of zeros, and the softmax maximum and
// reciprocal sum of each output pixel of the chunk.
__host__ __device__ inline uint32_t bin_lds_words(const BinGeo& b)
{
    return ((uint32_t)(2 * b.nb_max + 1 + 16) + 3u) & ~3u;
}
__host__ __device__ inline uint32_t bin_lds_bytes(const BinGeo& b)
{
    return bin_lds_words(b) * 4u + (uint32_t)b.cap * 16u +
           (uint32_t)((b.R * b.ew_max + 1) * bin_row_bytes(b.Cg, b.eb) + 8 * b.R * b.ew_max);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps
// within each row of 16 lanes (DPP row shifts by 1, 2, 4, 8; lanes shifted in
// from outside the row add 0), then the running total of row 0 broadcast
// into rows 1 and 3 and that of row 1 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// Exclusive prefix sums of cnt[0, nb) into start[0, nb] (start[nb] is the
// total), by the whole workgroup (NT threads, a multiple of 64).  Every
// thread takes a run of consecutive bins; the runs' sums are scanned within
// each wave and across waves through wsum.  Starts and ends with a barrier.
__device__ __forceinline__ void bin_scan(const uint32_t* cnt, uint32_t* start, uint32_t* wsum, int nb, int t, int NT)
{
    __syncthreads();
    const int per = (nb + NT - 1) / NT;
    const int b0 = t * per, b1 = b0 + per < nb ? b0 + per : nb;
    uint32_t local = 0;
    for (int b = b0; b < b1; ++b) local += cnt[b];
    const int lane = t & 63, wave = t >> 6;
    const uint32_t v = wave_inclusive_scan(local);
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    uint32_t run = base + v - local;
    for (int b = b0; b < b1; ++b) {
        start[b] = run;
        run += cnt[b];
    }
    if (t == NT - 1) start[nb] = base + v;
    __syncthreads();
}

// CPL gradient elements of a staged row, widened to binary32 (exactly).
template <typename T, int CPL>
__device__ __forceinline__ void load_grad_row(const char* p, float (&v)[CPL])
{
    if constexpr (Elem<T>::bytes == 4) {
#pragma unroll
        for (int c = 0; c < CPL / 4; ++c) {
            const float4 f = *(const float4*)(p + 16 * c);
            v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPL / 8; ++c) {
            const uint4 h = *(const uint4*)(p + 16 * c);
            const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[8 * c + 2 * q] = Elem<T>::widen(w[q] & 0xffffu);
                v[8 * c + 2 * q + 1] = Elem<T>::widen(w[q] >> 16);
            }
        }
    }
}

// Adds the records [e0, e2) of a run of two bins into acc: the records of the
// first bin [e0, e1) have this pixel as their right-hand corner (dx = 1), the
// others as their left-hand one; lower: the pixel is the lower corner
// (dy = 1) of all the run's records.  Two records per step, both gradient
// rows read before either is used; a run of odd length ends on a step whose
// second record has weight 0 and reads the zero row zr (a record's own row
// could hold an Inf, and 0 * Inf is not 0).
template <typename T, int CPL>
__device__ __forceinline__ void bin_run(const uint4* rec_lds, const char* gp, const char* zr, int e0, int e1,
                                        int e2, bool lower, float (&acc)[CPL])
{
#pragma unroll 1
    for (int e = e0; e < e2; e += 2) {
        const bool two = e + 1 < e2;
        const uint4 r0 = rec_lds[e];
        const uint4 r1 = rec_lds[two ? e + 1 : e];
        float v0[CPL], v1[CPL];
        load_grad_row<T, CPL>(gp + r0.x, v0);
        load_grad_row<T, CPL>(two ? gp + r1.x : zr, v1);
        const float wx0 = e < e1 ? __uint_as_float(r0.z) : 1.0f - __uint_as_float(r0.z);
        const float wx1 = e + 1 < e1 ? __uint_as_float(r1.z) : 1.0f - __uint_as_float(r1.z);
        const float wy0 = lower ? __uint_as_float(r0.w) : 1.0f - __uint_as_float(r0.w);
        const float wy1 = lower ? __uint_as_float(r1.w) : 1.0f - __uint_as_float(r1.w);
        const float w0 = __uint_as_float(r0.y) * (wy0 * wx0);
        const float w1 = two ? __uint_as_float(r1.y) * (wy1 * wx1) : 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w0, v0[c], acc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w1, v1[c], acc[c]);
    }
}

// T: element type; KT: K, or 0 for a runtime K; CPL: channels per gather
// lane (8 or 16, dividing Cg).  NT threads (a multiple of 64): every lane
// takes at most one (pixel, channel part) item of the tile, at most
// kBinSamples samples of a chunk and at most kBinPrefetch pieces of its
// gradient rows.
template <typename T, int KT, int CPL>
__global__ __launch_bounds__(1024) void dcn_backward_input_binned(BwdArgs a, BinGeo bg)
{
    constexpr int EB = Elem<T>::bytes;
    extern __shared__ uint4 bin_lds[];
    const Geometry& G = a.geo;
    const int t = threadIdx.x, NT = blockDim.x;
    uint32_t rest = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t tx = rest % bg.tiles_x;
    rest /= bg.tiles_x;
    const uint32_t ty = rest % bg.tiles_y;
    rest /= bg.tiles_y;
    const uint32_t g = rest % (uint32_t)G.groups;
    const uint32_t n = rest / (uint32_t)G.groups;
    const int qx0 = (int)tx * bg.TW, qy0 = (int)ty * bg.TH;
    const int tw = bg.TW < G.W - qx0 ? bg.TW : G.W - qx0;     // ragged last column / row of tiles
    const int th = bg.TH < G.H - qy0 ? bg.TH : G.H - qy0;
    const int nbx = tw + 1, nb = nbx * (th + 1);
    // Upstream-gradient rows are staged in binary32 (RE = 4: each bf16 element
    // is widened once per chunk rather than once per record that reads it),
    // fp16 ones as they are (the gather's mixed-precision FMA reads them
    // directly; binary32 rows measured 1% slower there, bf16 ones 6% faster).
    using RowT = typename std::conditional<Elem<T>::mixed_fma, T, float>::type;
    constexpr int RE = Elem<RowT>::bytes;
    const int RB = bin_row_bytes(bg.Cg, RE);

    uint32_t* cnt = (uint32_t*)bin_lds;
    uint32_t* start = cnt + bg.nb_max;
    uint32_t* wsum = start + bg.nb_max + 1;
    uint4* rec_lds = bin_lds + bin_lds_words(bg) / 4;
    char* gst = (char*)(rec_lds + bg.cap);
    char* zrow = gst + bg.R * bg.ew_max * RB;
    float2* smx = (float2*)(zrow + RB);

    // this lane's gather item: tile pixel (cx, cy), channels [part*CPL, +CPL)
    const int LP = bg.Cg / CPL;
    const bool has_item = t < th * tw * LP;
    const int ipx = t / LP, ipart = t - ipx * LP;
    const int icy = ipx / tw, icx = ipx - icy * tw;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

    int wlo, whi, hlo, hhi;
    owner_range(G, bg.M, qx0, tw, G.Wo, wlo, whi);
    owner_range(G, bg.M, qy0, th, G.Ho, hlo, hhi);
    const int EW = whi - wlo + 1;
    // Chunks interleave the visited rows (chunk k takes rows hlo + k,
    // hlo + k + nch, ...), so every chunk's samples spread over the whole tile
    // and each lane gathers a share of its records in every chunk, rather
    // than all of them in the one or two chunks whose rows lie over it.
    const int EH = EW > 0 && hhi >= hlo ? hhi - hlo + 1 : 0;
    const int nch = (EH + bg.R - 1) / bg.R;
    const int K = KT > 0 ? KT : G.K;
    const int P = KT > 0 ? KT * KT : G.P;
    const int centre = G.rc ? (K * K - 1) >> 1 : 1 << 30;     // the left-out tap, if any
    // Quotients of non-negative integers v by EW, P and K as
    // floor((v + 0.5) * (1/d)) in binary32: the true quotient is at least
    // 0.5/d away from an integer and the two roundings move it by less than
    // (v + 0.5)/d * 2^-23, which is smaller for v < 2^22 (here v < 2^13).
    const float inv_ew = EW > 0 ? 1.0f / (float)EW : 0.f, inv_p = 1.0f / (float)P, inv_k = 1.0f / (float)K;
    const uint32_t M2 = 2u * (uint32_t)bg.M;
    const RecordRsrc ro = record_rsrc((const char*)a.offset + (size_t)n * bg.off_image_bytes, bg.off_image_bytes);
    const RecordRsrc rm = record_rsrc((const char*)a.mask + (size_t)n * bg.mask_image_bytes, bg.mask_image_bytes);
    const bool odd = EB == 2 && (G.off_stride & 1);   // records on 2-byte boundaries
    const char* gout_img = (const char*)a.grad_out + (size_t)n * G.Ho * G.Wo * G.C * EB + g * bg.Cg * EB;
    const int pieces = bg.Cg * EB / 16;             // 16-byte pieces of a group's gradient row
    auto mval = [&](uint32_t raw) { return EB == 4 ? __uint_as_float(raw) : Elem<T>::widen(raw); };
    // (24-bit multiplies: the planner keeps Ho*Wo*G and the record and
    // pixel strides below 2^24)
    auto record_offset = [&](int kc, int e, uint32_t stride_bytes) {
        const int r = (int)(((float)e + 0.5f) * inv_ew), c = e - __mul24(r, EW);
        const uint32_t row = (uint32_t)(hlo + kc + __mul24(nch, r));
        const uint32_t pg_img = __umul24(__umul24(row, (uint32_t)G.Wo) + (uint32_t)(wlo + c), (uint32_t)G.groups) + g;
        return __umul24(pg_img, stride_bytes);
    };

    // A unit is NJ consecutive points of one output pixel: a row of the 3 x 3
    // taps (i fixed, j = 0, 1, 2) in the K = 3 specialisation, which shares
    // the pixel's decoding and loads its three offset pairs and mask values
    // with wide loads; a single point otherwise.  Lanes take units
    // u = t + k*NT, k < NUL (kBinSamples samples per lane either way).
    constexpr int NJ = KT > 0 ? KT : 1;
    constexpr int NUL = kBinSamples / NJ;
    static_assert(NUL * NJ == kBinSamples, "units per lane");
    const int UPP = P / NJ;                          // units per output pixel
    const float inv_upp = 1.0f / (float)UPP;

    // The loads of a chunk: units (their offset pairs and mask values) and
    // gradient pieces j = t + k*NT.  Every lane issues every load; those past
    // the chunk get an out-of-range offset and read zeros, so no branch
    // separates a load from the code that uses it.
    const __amdgpu_buffer_rsrc_t rg = image_rsrc(gout_img - g * bg.Cg * EB, bg.gout_image_bytes);
    const uint32_t gcol = g * (uint32_t)(bg.Cg * EB);
    const float inv_pieces = 1.0f / (float)pieces;
    uint32_t pd[NUL][NJ][EB == 4 ? 2 : 1];
    uint32_t pm[NUL][NJ];
    uint4 gpre[kBinPrefetch];
    auto prefetch = [&](int kc) {
        const int rows = kc < nch ? (EH - kc + nch - 1) / nch : 0;
        const int NU = rows * EW * UPP;
#pragma unroll
        for (int k = 0; k < NUL; ++k) {
            int u = t + k * NT;
            asm volatile("" : "+v"(u));     // decoded afresh each chunk (not held across the loop)
            const bool ok = u < NU;
            const int e = (int)(((float)u + 0.5f) * inv_upp), q0 = (u - __mul24(e, UPP)) * NJ;
            const uint32_t vo = ok ? record_offset(kc, e, (uint32_t)(G.off_stride * EB)) + ro.lead : kOOB;
            const uint32_t vm = ok ? record_offset(kc, e, (uint32_t)(G.mask_stride * EB)) + rm.lead : kOOB;
            if constexpr (EB == 4) {
                if constexpr (NJ == 3) {
                    const auto a4 = __builtin_amdgcn_raw_buffer_load_b128(ro.r, vo + 8u * (uint32_t)q0, 0, 0);
                    const auto a2 = __builtin_amdgcn_raw_buffer_load_b64(ro.r, vo + 8u * (uint32_t)q0 + 16u, 0, 0);
                    const auto m3 = __builtin_amdgcn_raw_buffer_load_b96(rm.r, vm + 4u * (uint32_t)q0, 0, 0);
                    pd[k][0][0] = a4[0]; pd[k][0][1] = a4[1];
                    pd[k][1][0] = a4[2]; pd[k][1][1] = a4[3];
                    pd[k][2][0] = a2[0]; pd[k][2][1] = a2[1];
                    pm[k][0] = m3[0]; pm[k][1] = m3[1]; pm[k][2] = m3[2];
                } else {
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) {
                        const uint32_t qq = (uint32_t)(q0 + jj);
                        const auto v = __builtin_amdgcn_raw_buffer_load_b64(ro.r, vo + 8u * qq, 0, 0);
                        pd[k][jj][0] = v[0];
                        pd[k][jj][1] = v[1];
                        pm[k][jj] = __builtin_amdgcn_raw_buffer_load_b32(rm.r, vm + 4u * qq, 0, 0);
                    }
                }
            } else {
                if (NJ == 3 && !odd) {
                    // three offset pairs on a 4-byte boundary
                    const auto a3 = __builtin_amdgcn_raw_buffer_load_b96(ro.r, vo + 4u * (uint32_t)q0, 0, 0);
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) pd[k][jj][0] = a3[jj < 3 ? jj : 0];
                } else {
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) {
                        const uint32_t o = vo + 4u * (uint32_t)(q0 + jj);
                        if (odd) {
                            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(ro.r, o, 0, 0);
                            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(ro.r, o + 2u, 0, 0);
                            pd[k][jj][0] = lo | (hi << 16);
                        } else {
                            pd[k][jj][0] = __builtin_amdgcn_raw_buffer_load_b32(ro.r, o, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj)
                    pm[k][jj] = __builtin_amdgcn_raw_buffer_load_b16(rm.r, vm + 2u * (uint32_t)(q0 + jj), 0, 0);
            }
        }
#pragma unroll
        for (int k = 0; k < kBinPrefetch; ++k) {
            int j = t + k * NT;
            asm volatile("" : "+v"(j));
            const int CP = rows * EW;
            const int e = (int)(((float)j + 0.5f) * inv_pieces), pc = j - __mul24(e, pieces);
            const int r = (int)(((float)e + 0.5f) * inv_ew), c = e - __mul24(r, EW);
            const uint32_t row = (uint32_t)(hlo + kc + __mul24(nch, r));
            const uint32_t off = j < CP * pieces
                                     ? __umul24(__umul24(row, (uint32_t)G.Wo) + (uint32_t)(wlo + c), (uint32_t)(G.C * EB)) +
                                           gcol + (uint32_t)pc * 16u
                                     : kOOB;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0);
            gpre[k] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };

    for (int b = t; b < nb; b += NT) cnt[b] = 0u;
    for (int c = t; c < RB / 4; c += NT) ((uint32_t*)zrow)[c] = 0u;
    prefetch(0);
    __syncthreads();

    for (int kc = 0; kc < nch; ++kc) {
        const int rows = (EH - kc + nch - 1) / nch;
        const int CP = rows * EW;

        // the chunk's upstream-gradient rows of this group, as they are
#pragma unroll
        for (int k = 0; k < kBinPrefetch; ++k) {
            const int j = t + k * NT;
            if (j < CP * pieces) {
                const int e = (int)(((float)j + 0.5f) * inv_pieces), pc = j - e * pieces;
                if constexpr (RE == EB) {
                    *(uint4*)(gst + e * RB + pc * 16) = gpre[k];
                } else {
                    const uint32_t w[4] = {gpre[k].x, gpre[k].y, gpre[k].z, gpre[k].w};
                    float f[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f[2 * q] = Elem<T>::widen(w[q] & 0xffffu);
                        f[2 * q + 1] = Elem<T>::widen(w[q] >> 16);
                    }
                    float4* dst = (float4*)(gst + e * RB + pc * 32);
                    dst[0] = make_float4(f[0], f[1], f[2], f[3]);
                    dst[1] = make_float4(f[4], f[5], f[6], f[7]);
                }
            }
        }
        if (G.softmax) {
            // the softmax of each output pixel's mask row, once per chunk
            for (int e = t; e < CP; e += NT) {
                const uint32_t vm = record_offset(kc, e, (uint32_t)(G.mask_stride * EB)) + rm.lead;
                float mx = load_mask_value<T>(rm.r, vm, 0);
                for (int q = 1; q < P; ++q) mx = fmaxf(mx, load_mask_value<T>(rm.r, vm, q));
                float sum = 0.f;
                for (int q = 0; q < P; ++q) sum += __expf(load_mask_value<T>(rm.r, vm, q) - mx);
                smx[e] = make_float2(mx, 1.0f / sum);
            }
            __syncthreads();
        }

        // Bin this lane's samples: an LDS atomic on the bin's count returns
        // the sample's slot in its bin, and after the scan its record goes to
        // the bin's start plus that slot.  (The slots are first used after
        // the scan, so the atomics' returns are waited for once, not one by
        // one.)
        const int NU = rows * EW * UPP;
        uint32_t sbin[NUL][NJ], sslot[NUL][NJ];   // bin (~0: no record) and slot
        float sw[NUL][NJ][3];                     // m, lx, ly
        const int base_off = G.c0 - G.pad;
#pragma unroll
        for (int k = 0; k < NUL; ++k) {
            int u = t + k * NT;
            asm volatile("" : "+v"(u));
            // every step computed for every lane, one predicate per sample
            const int e = (int)(((float)u + 0.5f) * inv_upp), iu = u - __mul24(e, UPP);
            const int r = (int)(((float)e + 0.5f) * inv_ew), c = e - __mul24(r, EW);
            const int bxi = __mul24(wlo + c, G.stride) + base_off;
            const float bxf = (float)bxi;
            const int byi = __mul24(hlo + kc + __mul24(nch, r), G.stride) + base_off;
            const float byf = (float)byi;
            float smx_m = 0.f, smx_inv = 1.f;
            if (G.softmax) {
                const float2 sm = smx[u < NU ? e : 0];
                smx_m = sm.x;
                smx_inv = sm.y;
            }
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                int i, j;
                if constexpr (KT > 0) {
                    i = iu;
                    j = jj;
                } else {
                    const int tap = iu + (iu >= centre ? 1 : 0);
                    i = (int)(((float)tap + 0.5f) * inv_k);
                    j = tap - __mul24(i, K);
                }
                float2 d;
                if constexpr (EB == 4) d = make_float2(__uint_as_float(pd[k][jj][0]), __uint_as_float(pd[k][jj][1]));
                else d = make_float2(Elem<T>::widen(pd[k][jj][0] & 0xffffu), Elem<T>::widen(pd[k][jj][0] >> 16));
                float m = mval(pm[k][jj]);
                if (G.softmax) m = __expf(m - smx_m) * smx_inv;
                const float x = fmaf(G.alpha, d.x, fmaf(G.alpha, (float)(__mul24(i, G.dil) - G.c0), bxf));
                const float y = fmaf(G.alpha, d.y, fmaf(G.alpha, (float)(__mul24(j, G.dil) - G.c0), byf));
                // the skip rule of the definition (false for NaN)
                const bool inmap = x > -1.0f && x < (float)G.W && y > -1.0f && y < (float)G.H;
                const float fx = floorf(inmap ? x : -2.0f), fy = floorf(inmap ? y : -2.0f);
                const int x0 = (int)fx, y0 = (int)fy;
                // near: both corners of each axis within M of the base
                const bool near = (uint32_t)(x0 - bxi + bg.M) < M2 && (uint32_t)(y0 - byi + bg.M) < M2;
                const int bx = x0 - qx0 + 1, by = y0 - qy0 + 1;      // bin coordinates
                const bool valid =
                    u < NU && inmap && near && (uint32_t)bx <= (uint32_t)tw && (uint32_t)by <= (uint32_t)th;
                const uint32_t bin = (uint32_t)(__mul24(by, nbx) + bx);
                sbin[k][jj] = valid ? bin : ~0u;
                sslot[k][jj] = 0u;
                if (valid) sslot[k][jj] = atomicAdd(cnt + bin, 1u);
                sw[k][jj][0] = m;
                sw[k][jj][1] = x - fx;
                sw[k][jj][2] = y - fy;
            }
        }
        bin_scan(cnt, start, wsum, nb, t, NT);
        // the counts are not read again in this chunk: clear them for the
        // next one (past the barriers below)
        for (int b = t; b < nb; b += NT) cnt[b] = 0u;
        uint32_t pos[NUL][NJ];
#pragma unroll
        for (int k = 0; k < NUL; ++k)
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
                pos[k][jj] = start[sbin[k][jj] == ~0u ? 0u : sbin[k][jj]] + sslot[k][jj];
#pragma unroll
        for (int k = 0; k < NUL; ++k) {
            int u = t + k * NT;
            asm volatile("" : "+v"(u));
            const uint32_t goff = (uint32_t)((int)(((float)u + 0.5f) * inv_upp) * RB);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
                if (sbin[k][jj] != ~0u && pos[k][jj] < (uint32_t)bg.cap)
                    rec_lds[pos[k][jj]] = make_uint4(goff, __float_as_uint(sw[k][jj][0]), __float_as_uint(sw[k][jj][1]),
                                                     __float_as_uint(sw[k][jj][2]));
        }
        __syncthreads();
        prefetch(kc + 1);

        // gather: the two runs of records of the item's 2x2 bins
        if (has_item) {
            const int bU = icy * nbx + icx, bL = bU + nbx;
            const char* gp = gst + ipart * CPL * RE;
            // (every start is at most the chunk's record count, which is
            // at most cap; the clamp keeps the reads inside the records
            // whatever the counts)
            const int cap = bg.cap;
            auto st = [&](int b) { const int v = (int)start[b]; return v < cap ? v : cap; };
            const char* zr = zrow + ipart * CPL * RE;
            bin_run<RowT, CPL>(rec_lds, gp, zr, st(bU), st(bU + 1), st(bU + 2), true, acc);
            bin_run<RowT, CPL>(rec_lds, gp, zr, st(bL), st(bL + 1), st(bL + 2), false, acc);
        }
        __syncthreads();
    }

    // write the tile, rounded once to the dtype
    if (has_item) {
        if (a.gi_init) {
            // add the binary32 partial sums already in the workspace (the
            // corners of samples that are not near)
            const float4* src = (const float4*)(a.gi_init + (size_t)n * G.H * G.W * G.C +
                                                ((size_t)(qy0 + icy) * G.W + (qx0 + icx)) * G.C + g * bg.Cg +
                                                ipart * CPL);
#pragma unroll
            for (int c = 0; c < CPL / 4; ++c) {
                const float4 v = src[c];
                acc[4 * c] = v.x + acc[4 * c];
                acc[4 * c + 1] = v.y + acc[4 * c + 1];
                acc[4 * c + 2] = v.z + acc[4 * c + 2];
                acc[4 * c + 3] = v.w + acc[4 * c + 3];
            }
        }
        char* dst = (char*)a.grad_input + (size_t)n * G.in_image_bytes + g * (bg.Cg * EB) +
                    (size_t)(qy0 + icy) * G.in_line_bytes + (size_t)(qx0 + icx) * G.in_row_bytes + ipart * (CPL * EB);
#pragma unroll
        for (int c = 0; c < CPL; c += 16 / EB) store<T, 16>(dst + c * EB, &acc[c]);
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
            // a skipped sample has zero gradients whatever its mask value
            if (!s.inmap) { gm = 0.f; gdx = 0.f; gdy = 0.f; }
            const float am = s.inmap ? G.alpha * m : 0.f;
            if (act && leader) {
                store_pair<T>(goff + 2 * p, am * gdx, am * gdy);
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
