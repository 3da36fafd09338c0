// dcn_core.hip -- C ABI of the deformable sampling core (declared in
// include/dcn_core.h): host-side validation, launch geometry and the choice
// of one template variant of each kernel.  The operation is defined in the
// header; the kernels live in dcn_kernels.hpp.
//
// Variants are compile-time specialisations of one kernel (element type,
// gather width, channels per lane, K = 3 or runtime K), chosen from the
// sizes and pointer alignment of the call; there is no other code path.

#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include <hip/hip_runtime.h>

#include "dcn_core.h"
#include "dcn_kernels.hpp"
#include "dcn_gate.hpp"
#include "dcn_linear.hpp"
#include "dcn_wgrad.hpp"

using namespace dcn;

namespace {

#ifndef DCN_USE_TILES
#define DCN_USE_TILES 1       // stage input tiles in LDS where the shape allows
#endif
#ifndef DCN_WIDE_ROWS
#define DCN_WIDE_ROWS 1   // one lane gathers a 32-byte group row as two 16-byte loads
#endif

constexpr int64_t kMaxImageBytes = (1ll << 31) - 4096;   // one image must fit a buffer resource

struct Call {
    int N, H, W, G, Cg, K, stride, pad, dil, Ho, Wo;
    float alpha;
    int softmax, dtype, ebytes;
    int rc;              // remove_center: the centre tap is left out
    int packed;          // offsets and mask share one record of 3P values per (pixel, group)
    int P;               // points per (pixel, group): K*K - rc
    int off_stride;      // elements per (pixel, group) record of the offset tensor
    int mask_stride;     // ... of the mask tensor (the packed record for both when packed)
    // The K = 3 specialisations index the full 3 x 3 grid at compile time.
    bool k3() const { return K == 3 && !rc; }
};

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int elem_bytes(int dtype)
{
    switch (dtype) {
    case DCN_F32: return 4;
    case DCN_F16: return 2;
    case DCN_BF16: return 2;
    default: return 0;
    }
}

// Host validation shared by forward and backward; touches no device state.
// remove_center needs an odd K >= 3; packed selects the one-record layout.
int validate(Call& c, int N, int H, int W, int G, int Cg, int K, int stride, int pad, int dil,
             float alpha, int softmax, int dtype, int remove_center = 0, int packed = 0)
{
    c = Call{N, H, W, G, Cg, K, stride, pad, dil, 0, 0, alpha, softmax, dtype, elem_bytes(dtype),
             remove_center, packed, 0, 0, 0};
    if (c.ebytes == 0) return DCN_ERR_INVALID_ARG;
    if (N < 0 || H < 1 || W < 1 || G < 1 || Cg < 1 || K < 1 || stride < 1 || dil < 1 || pad < 0)
        return DCN_ERR_INVALID_ARG;
    if (softmax != 0 && softmax != 1) return DCN_ERR_INVALID_ARG;
    if (remove_center != 0 && remove_center != 1) return DCN_ERR_INVALID_ARG;
    if (remove_center && (K % 2 == 0 || K < 3)) return DCN_ERR_INVALID_ARG;
    c.P = K * K - remove_center;
    c.off_stride = packed ? 3 * c.P : 2 * c.P;
    c.mask_stride = packed ? 3 * c.P : c.P;
    if (!(alpha == alpha) || alpha - alpha != 0.0f) return DCN_ERR_INVALID_ARG;   // NaN or Inf
    c.Ho = dcn_core_out_size(H, K, stride, pad, dil);
    c.Wo = dcn_core_out_size(W, K, stride, pad, dil);
    if (c.Ho <= 0 || c.Wo <= 0) return DCN_ERR_INVALID_ARG;
    if (K > 16) return DCN_ERR_UNSUPPORTED;
    const int64_t C = (int64_t)G * Cg;
    if (C >= (1ll << 31)) return DCN_ERR_UNSUPPORTED;
    const int64_t in_img = (int64_t)H * W * C, out_img = (int64_t)c.Ho * c.Wo * C;
    const int64_t off_img = (int64_t)c.Ho * c.Wo * G * c.off_stride;
    if (in_img * c.ebytes > kMaxImageBytes || out_img >= (1ll << 31) || off_img >= (1ll << 31))
        return DCN_ERR_UNSUPPORTED;
    return DCN_OK;
}

Geometry make_geometry(const Call& c, int cpl)
{
    Geometry g{};
    g.H = c.H; g.W = c.W; g.C = c.G * c.Cg; g.groups = c.G; g.Ho = c.Ho; g.Wo = c.Wo;
    g.K = c.K; g.P = c.P; g.stride = c.stride; g.pad = c.pad; g.dil = c.dil;
    g.c0 = c.dil * (c.K - 1) / 2;
    g.rc = c.rc;
    g.off_stride = c.off_stride;
    g.mask_stride = c.mask_stride;
    g.alpha = c.alpha;
    g.softmax = c.softmax;
    g.in_row_bytes = (uint32_t)(g.C * c.ebytes);
    g.in_line_bytes = (uint32_t)((int64_t)c.W * g.C * c.ebytes);
    g.in_image_bytes = (uint32_t)((int64_t)c.H * c.W * g.C * c.ebytes);
    const uint32_t chunks = (uint32_t)(g.C / cpl);
    g.lanes_per_image = (uint32_t)c.Ho * (uint32_t)c.Wo * chunks;
    g.blocks_per_image = (g.lanes_per_image + kBlock - 1) / kBlock;
    g.chunks = make_fastdiv(chunks);
    g.lanes_per_group = make_fastdiv((uint32_t)(c.Cg / cpl));
    g.wo_div = make_fastdiv((uint32_t)c.Wo);
    return g;
}

int launch_status()
{
    return hipGetLastError() == hipSuccess ? DCN_OK : DCN_ERR_HIP;
}

template <typename T, int LB, int NL>
int forward_variant(const FwdArgs& base, const Call& c, hipStream_t st)
{
    constexpr int CPL = NL * LB / (int)sizeof(T);
    FwdArgs a = base;
    a.geo = make_geometry(c, CPL);
    const uint64_t blocks = (uint64_t)c.N * a.geo.blocks_per_image;
    if (blocks >= (1ull << 31)) return DCN_ERR_UNSUPPORTED;
    if (c.k3())
        hipLaunchKernelGGL((dcn_forward_kernel<T, LB, NL, 3>), dim3((uint32_t)blocks), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((dcn_forward_kernel<T, LB, NL, 0>), dim3((uint32_t)blocks), dim3(kBlock), 0, st, a);
    return launch_status();
}

// ---------------------------------------------------------------- tiled path
#ifndef DCN_TILE_REACH
#define DCN_TILE_REACH 5      // offsets up to this many pixels stay inside the staged region
#endif
#ifndef DCN_TILE_FORCE_TW
#define DCN_TILE_FORCE_TW 0   // nonzero: fixed tile width (tuning builds)
#endif
#ifndef DCN_TILE_FORCE_TH
#define DCN_TILE_FORCE_TH 0
#endif
constexpr int64_t kMaxTileLds = 96 * 1024;
constexpr int kMaxTilePixels = 128;   // 512 lanes
// The forward planner may take a region of all of LDS with as few as 4
// resident waves per CU: measured on a stride-2 stage (bf16, 128x128 input,
// 512 channels), a 154 KB region with one block of 512 lanes per CU beats
// the direct gather by 1.5x (larger regions overfetch less at stride 2); the
// stride-1 stages keep their plans, which the cost model still prefers.
constexpr int64_t kMaxFwdTileLds = 160 * 1024;
constexpr int kMinFwdTileWaves = 4;

struct TilePlan {
    TileGeo tg;
    int threads;
    uint32_t lds_bytes;
    uint64_t blocks;
};

// The tiled kernel applies when a lane's 32 bytes never straddle two groups
// and 128-byte slabs tile the channel row: Cg*b in {32, 64, 128}, C*b a
// multiple of 128, 16-byte aligned input and output.  Among tile shapes with
// at most 128 pixels it picks the cheapest by a simple cost model: lane slots
// issued (idle lanes of ragged tiles count, weighted up below 16 resident
// waves per CU) plus region chunks staged; on equal cost the wider tile (a
// wave's pixels then span fewer tile rows; measured 1-3% faster at 56x56,
// 8x14 against 14x8).  A block has the lanes its tile needs (4 per pixel),
// rounded up to whole waves, so no wave runs without a pixel.  min_waves and
// max_lds are the caller's limits (the forward's are kMinFwdTileWaves and
// kMaxFwdTileLds); zero_block reserves the forward's 2x2 block of zero pixels
// after a partial region; reach is how far (pixels, before offset_scale)
// offsets may go and stay inside the staged region.
bool plan_tiles(const Call& c, const void* in, const void* out, TilePlan& plan, int min_waves = 12,
                int64_t max_lds = kMaxTileLds, bool zero_block = false, int reach = DCN_TILE_REACH)
{
    const int eb = c.ebytes, rowg = c.Cg * eb, rowc = c.G * c.Cg * eb;
    if (!(rowg == 32 || rowg == 64 || rowg == 128) || rowc % 128 != 0) return false;
    if (!aligned(in, 16) || !aligned(out, 16)) return false;
    if (c.stride > 4 || c.K * c.K > kMaxTiledTaps) return false;
    const int64_t off_img = (int64_t)c.Ho * c.Wo * c.G * c.off_stride * eb;
    const int64_t mask_img = (int64_t)c.Ho * c.Wo * c.G * c.mask_stride * eb;
    if (off_img >= (1ll << 31) || mask_img >= (1ll << 31)) return false;
    const float a = c.alpha < 0 ? -c.alpha : c.alpha;
    const int c0 = c.dil * (c.K - 1) / 2;
    const int span = c0 > c.dil * (c.K - 1) - c0 ? c0 : c.dil * (c.K - 1) - c0;
    const int ml = (int)ceilf(a * (float)span + a * (float)reach);
    const uint32_t slabs = (uint32_t)(rowc / 128);
    double best = -1.0;
    for (int tw = 1; tw <= 32 && tw <= c.Wo; ++tw) {
        for (int th = 1; th <= kMaxTilePixels / tw && th <= c.Ho; ++th) {
            if (DCN_TILE_FORCE_TW && (tw != DCN_TILE_FORCE_TW || th != DCN_TILE_FORCE_TH)) continue;
            // A region never needs more than the map and a one-pixel border
            // (tile_coord starts it no earlier than -1).  When that is all of
            // it on both axes the kernel reads no memory outside the region;
            // one more zero row then gives off-map samples a 2x2 block of
            // zeros to read.
            int rh = (th - 1) * c.stride + 2 * ml + 2, rw = (tw - 1) * c.stride + 2 * ml + 2;
            const bool whole = rh >= c.H + 2 && rw >= c.W + 2;
            if (rh > c.H + 2) rh = c.H + 2;
            if (rw > c.W + 2) rw = c.W + 2;
            if (whole) rh = c.H + 3;
            // the forward's block of zero pixels after a partial region (two
            // more rows' worth of address range, of which 2x2 pixels are used)
            const int64_t lds = ((int64_t)rh * rw + (zero_block && !whole ? rw + 2 : 0)) * 128;
            if (lds > max_lds) continue;
            const uint64_t tx = (uint64_t)((c.Wo + tw - 1) / tw), ty = (uint64_t)((c.Ho + th - 1) / th);
            const uint64_t tiles = tx * ty * slabs * (uint64_t)c.N;
            const int lanes = ((th * tw * 4 + 63) / 64) * 64;
            // LDS per block bounds the blocks a CU holds; below 16 resident
            // waves per CU the latency of the corner reads shows
            const int per_cu = (int)(160 * 1024 / lds) < 2048 / lanes ? (int)(160 * 1024 / lds) : 2048 / lanes;
            const int waves = per_cu * lanes / 64;
            if (waves < min_waves) continue;   // too few resident waves for this caller's kernel
            const double occ_penalty = waves >= 16 ? 1.0 : 16.0 / (double)waves;
            const double cost = (double)tiles * ((double)lanes * 900.0 * occ_penalty + (double)rh * rw * 8 * 3.0);
            if (best < 0 || cost < best || (cost == best && tw > plan.tg.TW)) {
                best = cost;
                plan.tg = TileGeo{th, tw, rh, rw, ml, 0, whole ? 1 : 0, (uint32_t)tx, (uint32_t)ty, slabs};
                plan.threads = lanes;
                plan.lds_bytes = (uint32_t)lds;
                plan.blocks = tiles;
            }
        }
    }
    if (best < 0 || plan.blocks >= (1ull << 31)) return false;
    int gs = 0;
    while ((32 << gs) < rowg) ++gs;
    plan.tg.gshift = gs;
    plan.tg.off_image_bytes = (uint32_t)off_img;
    plan.tg.mask_image_bytes = (uint32_t)mask_img;
    for (int i = 0, q = 0; i < c.K; ++i)
        for (int j = 0; j < c.K; ++j) {
            if (c.rc && i * c.K + j == (c.K * c.K - 1) / 2) continue;   // the left-out centre
            plan.tg.tap_x[q] = (float)(i * c.dil - c0);
            plan.tg.tap_y[q] = (float)(j * c.dil - c0);
            ++q;
        }
    return true;
}

template <typename T, int KT, int NT, bool SM, bool GATE = false>
int launch_tiled(const FwdArgs& a, const TilePlan& pl, hipStream_t st)
{
    // NT bounds the block; the block has the plan's lanes (whole waves)
    if (pl.tg.whole)
        hipLaunchKernelGGL((dcn_forward_tiled<T, KT, NT, SM, true, GATE>), dim3((uint32_t)pl.blocks),
                           dim3((uint32_t)pl.threads), pl.lds_bytes, st, a, pl.tg);
    else
        hipLaunchKernelGGL((dcn_forward_tiled<T, KT, NT, SM, false, GATE>), dim3((uint32_t)pl.blocks),
                           dim3((uint32_t)pl.threads), pl.lds_bytes, st, a, pl.tg);
    return launch_status();
}

template <typename T, int NT, bool SM>
int forward_tiled_k(const FwdArgs& a, const Call& c, const TilePlan& pl, hipStream_t st)
{
    return c.k3() ? launch_tiled<T, 3, NT, SM>(a, pl, st) : launch_tiled<T, 0, NT, SM>(a, pl, st);
}

template <typename T>
int forward_tiled(const FwdArgs& base, const Call& c, const TilePlan& pl, hipStream_t st)
{
    FwdArgs a = base;
    a.geo = make_geometry(c, 32 / (int)sizeof(T));
    if (a.gate) {   // raw mask only (the caller checks)
        if (pl.threads > 256)
            return c.k3() ? launch_tiled<T, 3, 512, false, true>(a, pl, st) : launch_tiled<T, 0, 512, false, true>(a, pl, st);
        return c.k3() ? launch_tiled<T, 3, 256, false, true>(a, pl, st) : launch_tiled<T, 0, 256, false, true>(a, pl, st);
    }
    if (pl.threads > 256)
        return c.softmax ? forward_tiled_k<T, 512, true>(a, c, pl, st) : forward_tiled_k<T, 512, false>(a, c, pl, st);
    return c.softmax ? forward_tiled_k<T, 256, true>(a, c, pl, st) : forward_tiled_k<T, 256, false>(a, c, pl, st);
}

// Widest gather whose size divides a group's row and whose alignment the
// input and output pointers allow; two 16-byte loads per corner when a
// group row holds 32 bytes or more.
template <typename T>
int forward_typed(const FwdArgs& a, const Call& c, hipStream_t st)
{
    TilePlan pl;
    if (DCN_USE_TILES && plan_tiles(c, a.input, a.output, pl, kMinFwdTileWaves, kMaxFwdTileLds, true))
        return forward_tiled<T>(a, c, pl, st);
    if (a.gate) return DCN_ERR_UNSUPPORTED;   // the gate is fused into the tiled kernel only
    const int row = c.Cg * (int)sizeof(T);
    auto ok = [&](int lb) {
        return row % lb == 0 && aligned(a.input, lb) && aligned(a.output, lb);
    };
    if (DCN_WIDE_ROWS && ok(16) && row % 32 == 0) return forward_variant<T, 16, 2>(a, c, st);
    if (ok(16)) return forward_variant<T, 16, 1>(a, c, st);
    if (ok(8)) return forward_variant<T, 8, 1>(a, c, st);
    if (ok(4)) return forward_variant<T, 4, 1>(a, c, st);
    if constexpr (sizeof(T) == 2) {
        if (ok(2)) return forward_variant<T, 2, 1>(a, c, st);
    }
    return DCN_ERR_INVALID_ARG;   // pointers not aligned to their element size
}

// ------------------------------------------------------ backward, owner tiles
#ifndef DCN_USE_OWNER
#define DCN_USE_OWNER 1       // grad_input by owner tiles where the shape allows
#endif
#ifndef DCN_OWNER_REACH
#define DCN_OWNER_REACH 5     // corners of offsets up to this many pixels are added by owners
#endif
#ifndef DCN_OWNER_FORCE_TW
#define DCN_OWNER_FORCE_TW 0  // nonzero: the owner planner considers only this tile (tuning builds)
#endif
#ifndef DCN_OWNER_FORCE_TH
#define DCN_OWNER_FORCE_TH 0
#endif
#ifndef DCN_OWNER_FORCE_R
#define DCN_OWNER_FORCE_R 0   // nonzero: ... and this many output rows per chunk
#endif
#ifndef DCN_OWNER_CHUNK_CLK
#define DCN_OWNER_CHUNK_CLK 1500   // modelled fixed cost of one chunk (barriers, scan), in lane-sample units
#endif
constexpr int64_t kMaxOwnerLds = 160 * 1024;
constexpr int kOwnerMaxTile = 32;
constexpr int kOwnerVgprs = 124;   // registers of the owner kernel per lane, at most (for the occupancy model)

struct OwnerPlan {
    BinGeo bg;
    int threads;
    int cpl;
    uint32_t lds_bytes;
    uint64_t blocks;
};

// The owner kernel applies where a group's channels split into lanes of 16
// or 8 (Cg a multiple of 8), with 16-byte aligned grad_output and grad_input.
// Among tiles up to 32 x 32 it picks the one with the least modelled work per
// CU (256 CUs): the samples its lanes bin, the records its items gather and a
// fixed cost per chunk, with a discount where two or more workgroups fit a
// CU (the measured effect of overlapping one's barriers with another's work).
bool plan_owner(const Call& c, const void* gout, const void* gin, OwnerPlan& pl)
{
    if (c.Cg % 8 != 0) return false;
    if (!aligned(gout, 16) || !aligned(gin, 16)) return false;
    const float a = c.alpha < 0 ? -c.alpha : c.alpha;
    const int c0 = c.dil * (c.K - 1) / 2;
    const int span = c0 > c.dil * (c.K - 1) - c0 ? c0 : c.dil * (c.K - 1) - c0;
    const float mf = ceilf(a * ((float)span + (float)DCN_OWNER_REACH)) + 1.0f;
    if (!(mf <= 1024.0f)) return false;
    const int M = (int)mf;
    const int cpl = c.Cg % 16 == 0 ? 16 : 8;
    const int LP = c.Cg / cpl;
    double best = -1.0;
    for (int tw = 1; tw <= kOwnerMaxTile && tw <= c.W; ++tw)
        for (int th = 1; th <= kOwnerMaxTile && th <= c.H; ++th) {
            if (DCN_OWNER_FORCE_TW && (tw != DCN_OWNER_FORCE_TW || th != DCN_OWNER_FORCE_TH)) continue;
            const int items = th * tw * LP;
            const int64_t tx = (c.W + tw - 1) / tw, ty = (c.H + th - 1) / th;
            int64_t ew = (tw - 1 + 2 * M) / c.stride + 1, eh = (th - 1 + 2 * M) / c.stride + 1;
            if (ew > c.Wo) ew = c.Wo;
            if (eh > c.Ho) eh = c.Ho;
            // visited output pixels over output pixels: beyond 8x the atomic
            // scatter is cheaper (a very large offset_scale makes every
            // output pixel near every tile)
            if ((double)(tx * ty) * (double)(ew * eh) > 8.0 * (double)c.Ho * c.Wo) continue;
            const int64_t blocks = tx * ty * (int64_t)c.G * c.N;
            if (blocks >= (1ll << 31)) continue;
            // one item per lane
            const int nt = (items + 63) / 64 * 64;
            if (nt > 1024) continue;
            for (int R = 1; R <= eh; ++R) {
                if (DCN_OWNER_FORCE_R && R != DCN_OWNER_FORCE_R) continue;
                BinGeo bg{th, tw, M, c.Cg, R, (int)ew, (int)(R * ew * c.P), (th + 1) * (tw + 1), 0u, 0u, 0u, 0u, 0u,
                          c.dtype == DCN_F16 ? 2 : 4};   // staged gradient rows: fp16, else binary32
                // a lane holds at most kBinSamples samples of a chunk and
                // kBinPrefetch 16-byte pieces of its gradient rows
                if (R * ew * c.P > kBinSamples * nt || R * ew * (c.Cg * c.ebytes / 16) > kBinPrefetch * nt) break;
                const int64_t lds = bin_lds_bytes(bg);
                if (lds > kMaxOwnerLds) break;
                const int waves = nt / 64;
                int bpc = (int)(kMaxOwnerLds / lds);
                const int by_waves = 32 / waves, by_regs = (512 / kOwnerVgprs) * 4 / waves;
                if (bpc > by_waves) bpc = by_waves;
                if (bpc > by_regs) bpc = by_regs;
                if (bpc < 1) continue;
                const int64_t chunks = (eh + R - 1) / R;
                // per CU: every lane bins kBinSamples samples per chunk, every
                // item gathers about 4P records, and each chunk pays a fixed
                // latency (barriers, scan); two or more resident workgroups
                // overlap one's barriers with another's work
                const double per_cu = (double)((blocks + 255) / 256);
                const double work = (double)chunks * nt * kBinSamples + (double)items * 4.0 * c.P * 0.8 +
                                    (double)chunks * DCN_OWNER_CHUNK_CLK;
                const double cost = per_cu * work / (bpc >= 2 ? 1.3 : 1.0);
                if (best < 0 || cost < best) {
                    best = cost;
                    pl.bg = bg;
                    pl.bg.tiles_x = (uint32_t)tx;
                    pl.bg.tiles_y = (uint32_t)ty;
                    pl.threads = nt;
                    pl.cpl = cpl;
                    pl.lds_bytes = (uint32_t)lds;
                    pl.blocks = (uint64_t)blocks;
                }
            }
        }
    if (best < 0) return false;
    const int64_t off_img = (int64_t)c.Ho * c.Wo * c.G * c.off_stride * c.ebytes;
    const int64_t mask_img = (int64_t)c.Ho * c.Wo * c.G * c.mask_stride * c.ebytes;
    const int64_t gout_img = (int64_t)c.Ho * c.Wo * c.G * c.Cg * c.ebytes;
    if (off_img >= (1ll << 31) || mask_img >= (1ll << 31) || gout_img >= (1ll << 31)) return false;
    // the kernel's 24-bit index products
    if ((int64_t)c.Ho * c.Wo * c.G >= (1 << 24) || (int64_t)c.G * c.Cg * c.ebytes >= (1 << 24) ||
        (int64_t)c.off_stride * c.ebytes >= (1 << 24))
        return false;
    pl.bg.off_image_bytes = (uint32_t)off_img;
    pl.bg.mask_image_bytes = (uint32_t)mask_img;
    pl.bg.gout_image_bytes = (uint32_t)gout_img;
    return true;
}

template <typename T, int KT>
int launch_owner(const BwdArgs& a, const OwnerPlan& pl, hipStream_t st)
{
    if (pl.cpl == 16)
        hipLaunchKernelGGL((dcn_backward_input_binned<T, KT, 16>), dim3((uint32_t)pl.blocks), dim3(pl.threads),
                           pl.lds_bytes, st, a, pl.bg);
    else
        hipLaunchKernelGGL((dcn_backward_input_binned<T, KT, 8>), dim3((uint32_t)pl.blocks), dim3(pl.threads),
                           pl.lds_bytes, st, a, pl.bg);
    return launch_status();
}

#ifndef DCN_USE_GRAD_TILES
#define DCN_USE_GRAD_TILES 1  // grad_offset / grad_mask from staged input tiles where the shape allows
#endif
#ifndef DCN_GRAD_TILE_REACH
#define DCN_GRAD_TILE_REACH 3 // the gradient kernel's region reach (its samples beyond it read global memory)
#endif

bool plan_grad_tiles(const Call& c, const void* in, const void* gout, TilePlan& tp, int min_waves = 12,
                     int64_t max_lds = kMaxTileLds)
{
    return plan_tiles(c, in, gout, tp, min_waves, max_lds, false, DCN_GRAD_TILE_REACH);
}

template <typename T, int KT, int NT>
int launch_grad_tiled(const BwdArgs& a, const Call& c, const TilePlan& pl, hipStream_t st)
{
    if (c.softmax)
        hipLaunchKernelGGL((dcn_backward_grad_tiled<T, KT, NT, true>), dim3((uint32_t)pl.blocks),
                           dim3((uint32_t)pl.threads), pl.lds_bytes, st, a, pl.tg);
    else
        hipLaunchKernelGGL((dcn_backward_grad_tiled<T, KT, NT, false>), dim3((uint32_t)pl.blocks),
                           dim3((uint32_t)pl.threads), pl.lds_bytes, st, a, pl.tg);
    return launch_status();
}

template <typename T>
int backward_grad_tiled(const BwdArgs& base, const Call& c, const TilePlan& pl, hipStream_t st)
{
    BwdArgs a = base;
    a.geo = make_geometry(c, 32 / (int)sizeof(T));
    if (pl.threads > 256)
        return c.k3() ? launch_grad_tiled<T, 3, 512>(a, c, pl, st) : launch_grad_tiled<T, 0, 512>(a, c, pl, st);
    return c.k3() ? launch_grad_tiled<T, 3, 256>(a, c, pl, st) : launch_grad_tiled<T, 0, 256>(a, c, pl, st);
}

int zero_fill(float* p, int64_t n, hipStream_t st);

// Half precision on the tiled shapes, every grad_input element a binary32 sum
// rounded once: the workspace (a binary32 image of grad_input) is zeroed, the
// tiled gradient kernel writes grad_offset and grad_mask and adds the corners
// beyond the owners' reach into the workspace, and the owner kernel starts
// its tiles from the workspace, adds the near corners and stores each
// element once in the dtype.
template <typename T>
int backward_half(BwdArgs a, const Call& c, float* ws, hipStream_t st)
{
    OwnerPlan op;
    TilePlan tp;
    // there is no untiled half-precision gradient kernel to fall back on, so
    // any tile that fits the LDS will do
    if (!plan_owner(c, a.grad_out, a.grad_input, op) || !plan_grad_tiles(c, a.input, a.grad_out, tp, 1, 160 * 1024))
        return DCN_ERR_UNSUPPORTED;
    int rc = zero_fill(ws, (int64_t)c.N * c.H * c.W * c.G * c.Cg, st);
    if (rc != DCN_OK) return rc;
    a.near_m = op.bg.M;
    a.far_ws = ws;
    rc = backward_grad_tiled<T>(a, c, tp, st);
    if (rc != DCN_OK) return rc;
    a.geo = make_geometry(c, 8);
    a.gi_init = ws;
    return c.k3() ? launch_owner<T, 3>(a, op, st) : launch_owner<T, 0>(a, op, st);
}

// Whether the tiled half-precision kernels take this call (both planners
// accept it); otherwise the untiled workspace kernel runs it.
bool half_tiled_ok(const Call& c, const void* input, const void* gout, const void* gin)
{
    OwnerPlan op;
    TilePlan tp;
    return plan_owner(c, gout, gin, op) && plan_grad_tiles(c, input, gout, tp, 1, 160 * 1024);
}

// Half-precision backward on any shape whose group splits into a power of
// two of lanes: binary32 atomics into the zeroed workspace, then one
// rounding into grad_input.
template <typename T>
int backward_generic(const BwdArgs& base, const Call& c, float* ws, hipStream_t st)
{
    const int eb = (int)sizeof(T);
    int lb = 0, L = 0;
    for (int cand = 16; cand >= eb; cand >>= 1) {
        const int cpl = cand / eb;
        if (c.Cg % cpl) continue;
        const int l = c.Cg / cpl;
        if (!(l > 0 && (l & (l - 1)) == 0 && l <= 64)) continue;
        if (!aligned(base.input, (uintptr_t)cand) || !aligned(base.grad_out, (uintptr_t)eb)) continue;
        lb = cand;
        L = l;
        break;
    }
    if (lb == 0) return DCN_ERR_UNSUPPORTED;
    const int64_t n = (int64_t)c.N * c.H * c.W * c.G * c.Cg;
    int rc = zero_fill(ws, n, st);
    if (rc != DCN_OK) return rc;
    BwdArgs a = base;
    a.geo = make_geometry(c, lb / eb);
    const uint64_t blocks = (uint64_t)c.N * a.geo.blocks_per_image;
    if (blocks >= (1ll << 31)) return DCN_ERR_UNSUPPORTED;
    const dim3 grid((uint32_t)blocks), blk(kBlock);
    const bool k3 = c.k3();
    switch (lb) {
    case 16:
        if (k3) hipLaunchKernelGGL((dcn_backward_generic<T, 16, 3>), grid, blk, 0, st, a, ws, L);
        else hipLaunchKernelGGL((dcn_backward_generic<T, 16, 0>), grid, blk, 0, st, a, ws, L);
        break;
    case 8:
        if (k3) hipLaunchKernelGGL((dcn_backward_generic<T, 8, 3>), grid, blk, 0, st, a, ws, L);
        else hipLaunchKernelGGL((dcn_backward_generic<T, 8, 0>), grid, blk, 0, st, a, ws, L);
        break;
    case 4:
        if (k3) hipLaunchKernelGGL((dcn_backward_generic<T, 4, 3>), grid, blk, 0, st, a, ws, L);
        else hipLaunchKernelGGL((dcn_backward_generic<T, 4, 0>), grid, blk, 0, st, a, ws, L);
        break;
    default:
        if (k3) hipLaunchKernelGGL((dcn_backward_generic<T, 2, 3>), grid, blk, 0, st, a, ws, L);
        else hipLaunchKernelGGL((dcn_backward_generic<T, 2, 0>), grid, blk, 0, st, a, ws, L);
        break;
    }
    rc = launch_status();
    if (rc != DCN_OK) return rc;
    const int64_t sb = (n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(dcn_store_workspace<T>, dim3((uint32_t)(sb < 4096 ? sb : 4096)), blk, 0, st, (const float*)ws,
                       (T*)a.grad_input, (size_t)n);
    return launch_status();
}

template <int LB, int L>
int backward_variant(const BwdArgs& base, const Call& c, hipStream_t st)
{
    BwdArgs a = base;
    a.geo = make_geometry(c, LB / 4);
    const uint64_t blocks = (uint64_t)c.N * a.geo.blocks_per_image;
    if (blocks >= (1ll << 31)) return DCN_ERR_UNSUPPORTED;
    if (c.k3())
        hipLaunchKernelGGL((dcn_backward_kernel<LB, L, 3>), dim3((uint32_t)blocks), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((dcn_backward_kernel<LB, L, 0>), dim3((uint32_t)blocks), dim3(kBlock), 0, st, a);
    return launch_status();
}

template <int LB>
int backward_lanes(const BwdArgs& a, const Call& c, hipStream_t st, int L)
{
    switch (L) {
    case 1: return backward_variant<LB, 1>(a, c, st);
    case 2: return backward_variant<LB, 2>(a, c, st);
    case 4: return backward_variant<LB, 4>(a, c, st);
    case 8: return backward_variant<LB, 8>(a, c, st);
    case 16: return backward_variant<LB, 16>(a, c, st);
    case 32: return backward_variant<LB, 32>(a, c, st);
    case 64: return backward_variant<LB, 64>(a, c, st);
    default: return DCN_ERR_UNSUPPORTED;
    }
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int zero_fill(float* p, int64_t n, hipStream_t st)
{
    if (n <= 0) return DCN_OK;
    int64_t head = 0;
    while (head < n && !aligned(p + head, 16)) ++head;   // at most 3 floats
    const int64_t n4 = (n - head) / 4;
    const int64_t tail = (n - head) - 4 * n4;
    // head and tail floats (at most 3 + 3) are written by block 0
    if (head > 0)
        hipLaunchKernelGGL(dcn_zero_kernel, dim3(1), dim3(kBlock), 0, st, (float4*)nullptr, (size_t)0, p,
                           (int)head);
    const int64_t blocks = n4 > 0 ? (n4 + kBlock - 1) / kBlock : 1;
    hipLaunchKernelGGL(dcn_zero_kernel, dim3((uint32_t)(blocks < 4096 ? blocks : 4096)), dim3(kBlock), 0, st,
                       (float4*)(p + head), (size_t)n4, p + head + 4 * n4, (int)tail);
    return launch_status();
}

}  // namespace

extern "C" int dcn_core_out_size(int in, int K, int stride, int pad, int dilation)
{
    if (in < 1 || K < 1 || stride < 1 || pad < 0 || dilation < 1) return 0;
    const int64_t span = (int64_t)dilation * (K - 1) + 1;
    const int64_t num = (int64_t)in + 2ll * pad - span;
    if (num < 0) return 0;
    const int64_t out = num / stride + 1;
    return out < (1ll << 31) ? (int)out : 0;
}

namespace {

// Flags of the _ex entry points -> validated call.
int validate_ex(Call& c, int N, int H, int W, int G, int Cg, int K, int stride, int pad, int dil,
                float alpha, int flags, int dtype)
{
    if (flags & ~(DCN_FLAG_SOFTMAX | DCN_FLAG_REMOVE_CENTER | DCN_FLAG_PACKED)) return DCN_ERR_INVALID_ARG;
    return validate(c, N, H, W, G, Cg, K, stride, pad, dil, alpha, (flags & DCN_FLAG_SOFTMAX) ? 1 : 0, dtype,
                    (flags & DCN_FLAG_REMOVE_CENTER) ? 1 : 0, (flags & DCN_FLAG_PACKED) ? 1 : 0);
}

// Pointer checks shared by both layouts.  A split offset record is a whole
// number of (dx, dy) pairs, so its base needs pair alignment; a packed record
// (3P values) only needs the tensor to start on a 4-byte boundary, the kernels
// realign records that fall on 2-byte boundaries.  The mask of a packed call
// is the record's tail, 2P elements in.
int resolve_records(const Call& c, const void* offset, const void* mask, const void** offset_out,
                    const void** mask_out)
{
    const uintptr_t eb = (uintptr_t)c.ebytes;
    if (c.packed) {
        if (mask || !aligned(offset, 4)) return DCN_ERR_INVALID_ARG;
        *offset_out = offset;
        *mask_out = (const char*)offset + (size_t)2 * c.P * c.ebytes;
    } else {
        if (!mask || !aligned(offset, 2 * eb) || !aligned(mask, eb)) return DCN_ERR_INVALID_ARG;
        *offset_out = offset;
        *mask_out = mask;
    }
    return DCN_OK;
}

int forward_call(const Call& c, const void* input, const void* offset, const void* mask, void* output,
                 void* stream, const void* gate = nullptr, void* core_out = nullptr)
{
    if (c.N == 0) return DCN_OK;
    if (!input || !offset || !output) return DCN_ERR_INVALID_ARG;
    FwdArgs a{};
    const int rc = resolve_records(c, offset, mask, &a.offset, &a.mask);
    if (rc != DCN_OK) return rc;
    a.input = input; a.output = output;
    a.gate = gate; a.core_out = core_out;
    hipStream_t st = (hipStream_t)stream;
    switch (c.dtype) {
    case DCN_F32: return forward_typed<float>(a, c, st);
    case DCN_F16: return forward_typed<_Float16>(a, c, st);
    default: return forward_typed<__bf16>(a, c, st);
    }
}

int backward_call(const Call& c, const void* input, const void* offset_in, const void* mask_in,
                  const void* grad_output, void* grad_input, void* grad_offset_in, void* grad_mask_in,
                  void* stream, void* workspace = nullptr, long long workspace_bytes = 0)
{
    const int N = c.N, H = c.H, W = c.W, G = c.G, Cg = c.Cg;
    if (N == 0) return DCN_OK;
    if (!input || !offset_in || !grad_output || !grad_input || !grad_offset_in) return DCN_ERR_INVALID_ARG;
    const void *offset, *mask, *grad_offset_c, *grad_mask_c;
    int rc = resolve_records(c, offset_in, mask_in, &offset, &mask);
    if (rc != DCN_OK) return rc;
    rc = resolve_records(c, grad_offset_in, grad_mask_in, &grad_offset_c, &grad_mask_c);
    if (rc != DCN_OK) return rc;
    void* grad_offset = const_cast<void*>(grad_offset_c);
    void* grad_mask = const_cast<void*>(grad_mask_c);
    const uintptr_t eb = (uintptr_t)c.ebytes;
    if (!aligned(input, eb) || !aligned(grad_output, eb) || !aligned(grad_input, eb)) return DCN_ERR_INVALID_ARG;
    const int dtype = c.dtype;
    if (dtype != DCN_F32) {
        // half precision accumulates grad_input in a binary32 workspace
        if (!workspace) return DCN_ERR_UNSUPPORTED;
        if (workspace_bytes < (long long)N * H * W * G * Cg * 4 || !aligned(workspace, 16)) return DCN_ERR_INVALID_ARG;
        BwdArgs a{};
        a.input = input; a.offset = offset; a.mask = mask; a.grad_out = grad_output;
        a.grad_input = grad_input; a.grad_offset = grad_offset; a.grad_mask = grad_mask;
        a.near_m = -1;
        hipStream_t st = (hipStream_t)stream;
        float* ws = (float*)workspace;
        if (half_tiled_ok(c, input, grad_output, grad_input))
            return dtype == DCN_F16 ? backward_half<_Float16>(a, c, ws, st) : backward_half<__bf16>(a, c, ws, st);
        return dtype == DCN_F16 ? backward_generic<_Float16>(a, c, ws, st) : backward_generic<__bf16>(a, c, ws, st);
    }
    int LB, L;
    if (Cg % 4 == 0 && pow2(Cg / 4) && Cg / 4 <= 64 && aligned(input, 16) && aligned(grad_input, 16)) {
        LB = 16; L = Cg / 4;
    } else if (pow2(Cg) && Cg <= 64) {
        LB = 4; L = Cg;
    } else {
        return DCN_ERR_UNSUPPORTED;
    }
    hipStream_t st = (hipStream_t)stream;
    BwdArgs a{};
    a.input = input; a.offset = offset; a.mask = mask; a.grad_out = grad_output;
    a.grad_input = grad_input; a.grad_offset = grad_offset; a.grad_mask = grad_mask;
    a.near_m = -1;
    OwnerPlan op;
    if (DCN_USE_OWNER && plan_owner(c, grad_output, grad_input, op)) {
        // owners write every element of grad_input; the gradient kernel
        // then adds the corners that are not near with atomics
        a.geo = make_geometry(c, 8);
        rc = c.k3() ? launch_owner<float, 3>(a, op, st) : launch_owner<float, 0>(a, op, st);
        a.near_m = op.bg.M;
    } else {
        rc = zero_fill((float*)grad_input, (int64_t)N * H * W * G * Cg, st);
    }
    if (rc != DCN_OK) return rc;
    TilePlan tp;
    if (DCN_USE_GRAD_TILES && plan_grad_tiles(c, input, grad_output, tp)) return backward_grad_tiled<float>(a, c, tp, st);
    return LB == 16 ? backward_lanes<16>(a, c, st, L) : backward_lanes<4>(a, c, st, L);
}
}  // namespace

extern "C" int dcn_core_forward_ex(const void* input, const void* offset, const void* mask, void* output,
                                   int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                                   int dilation, float offset_scale, int flags, int dtype, void* stream)
{
    Call c;
    const int rc = validate_ex(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, flags, dtype);
    if (rc != DCN_OK) return rc;
    return forward_call(c, input, offset, mask, output, stream);
}

extern "C" int dcn_core_forward_gated(const void* input, const void* offset, const void* mask,
                                      const void* gate_logits, void* output, void* core_output, int N, int H,
                                      int W, int G, int Cg, int K, int stride, int pad, int dilation,
                                      float offset_scale, int flags, int dtype, void* stream)
{
    Call c;
    const int rc = validate_ex(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, flags, dtype);
    if (rc != DCN_OK) return rc;
    // the output pixel's own input pixel is the centre of its taps: odd K,
    // stride 1, pad = dilation (K - 1) / 2; a raw mask
    if (K % 2 == 0 || stride != 1 || pad != dilation * (K - 1) / 2 || c.softmax) return DCN_ERR_UNSUPPORTED;
    if (N == 0) return DCN_OK;
    if (!gate_logits || !aligned(gate_logits, (uintptr_t)c.ebytes) ||
        (core_output && !aligned(core_output, 16)))
        return DCN_ERR_INVALID_ARG;
    return forward_call(c, input, offset, mask, output, stream, gate_logits, core_output);
}

extern "C" int dcn_core_forward(const void* input, const void* offset, const void* mask, void* output,
                                int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                                int dilation, float offset_scale, int softmax_flag, int dtype,
                                void* stream)
{
    Call c;
    const int rc = validate(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, softmax_flag, dtype);
    if (rc != DCN_OK) return rc;
    if (N > 0 && !mask) return DCN_ERR_INVALID_ARG;
    return forward_call(c, input, offset, mask, output, stream);
}

extern "C" int dcn_core_backward_ex(const void* input, const void* offset, const void* mask,
                                    const void* grad_output, void* grad_input, void* grad_offset,
                                    void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                                    int pad, int dilation, float offset_scale, int flags, int dtype,
                                    void* stream)
{
    Call c;
    const int rc = validate_ex(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, flags, dtype);
    if (rc != DCN_OK) return rc;
    return backward_call(c, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask, stream);
}

extern "C" long long dcn_core_backward_workspace_size(const void* input, const void* grad_output,
                                                      const void* grad_input, int N, int H, int W, int G, int Cg,
                                                      int K, int stride, int pad, int dilation, float offset_scale,
                                                      int flags, int dtype)
{
    Call c;
    const int rc = validate_ex(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, flags, dtype);
    if (rc != DCN_OK) return -(long long)rc;
    (void)input; (void)grad_output; (void)grad_input;
    if (dtype == DCN_F32 || N == 0) return 0;
    return (long long)N * H * W * G * Cg * 4;
}

extern "C" int dcn_core_backward_ws(const void* input, const void* offset, const void* mask,
                                    const void* grad_output, void* grad_input, void* grad_offset,
                                    void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                                    int pad, int dilation, float offset_scale, int flags, int dtype,
                                    void* workspace, long long workspace_bytes, void* stream)
{
    Call c;
    const int rc = validate_ex(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, flags, dtype);
    if (rc != DCN_OK) return rc;
    if (workspace_bytes < 0) return DCN_ERR_INVALID_ARG;
    return backward_call(c, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask, stream,
                         workspace, workspace_bytes);
}

extern "C" int dcn_core_backward(const void* input, const void* offset, const void* mask,
                                 const void* grad_output, void* grad_input, void* grad_offset,
                                 void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                                 int pad, int dilation, float offset_scale, int softmax_flag, int dtype,
                                 void* stream)
{
    Call c;
    const int rc = validate(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, softmax_flag, dtype);
    if (rc != DCN_OK) return rc;
    if (N > 0 && (!mask || !grad_mask)) return DCN_ERR_INVALID_ARG;
    return backward_call(c, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask, stream);
}

// ---------------------------------------------------------------------------
// dcn_core_backward_static: dcn_core_backward_ws with a fixed device array as
// its workspace, for callers that cannot allocate.  Each GPU the library runs
// on holds its own copy of the array until the process ends.  Host code must
// not pass `scratch` itself to a kernel (its host-side name is not a device
// address); the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that pointer is used.
constexpr long long kScratchBytes = DCN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxScratchDevices];   // device address of `scratch`, per device

// The current device's copy of the array (looked up on its first use there).
int device_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DCN_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return DCN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DCN_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return DCN_OK;
}
}  // namespace

extern "C" int dcn_core_backward_static(const void* input, const void* offset, const void* mask,
                                        const void* grad_output, void* grad_input, void* grad_offset,
                                        void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                                        int pad, int dilation, float offset_scale, int flags, int dtype,
                                        void* stream)
{
    Call c;
    const int rc = validate_ex(c, N, H, W, G, Cg, K, stride, pad, dilation, offset_scale, flags, dtype);
    if (rc != DCN_OK) return rc;
    if (dtype == DCN_F32 || N == 0)   // no workspace needed
        return backward_call(c, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask, stream);
    const long long need = (long long)N * H * W * G * Cg * 4;
    if (need > kScratchBytes) return DCN_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    const int src = device_scratch(&ws);
    if (src != DCN_OK) return src;
    return backward_call(c, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask, stream, ws,
                         kScratchBytes);
}

extern "C" const char* dcn_status_string(int status)
{
    switch (status) {
    case DCN_OK: return "DCN_OK";
    case DCN_ERR_INVALID_ARG: return "DCN_ERR_INVALID_ARG: invalid size, geometry, dtype, pointer or alignment";
    case DCN_ERR_UNSUPPORTED: return "DCN_ERR_UNSUPPORTED: valid request outside what this build implements";
    case DCN_ERR_HIP: return "DCN_ERR_HIP: the HIP runtime reported an error";
    case DCN_ERR_SCRATCH_LIMIT:
        return "DCN_ERR_SCRATCH_LIMIT: the call needs more than the library's static scratch "
               "(DCN_STATIC_SCRATCH_BYTES); use dcn_core_backward_ws";
    default: return "unknown dcn_status";
    }
}

// ---------------------------------------------------------------------------
// Centre-feature gate of the DCNv4 layer (dcn_gate.hpp).
namespace {

struct GateCall {
    uint64_t rows;
    uint32_t row_bytes;
    int vb;            // 16-byte vectors, or one element per access
    unsigned blocks;
};

int gate_validate(GateCall& gc, long long M, int G, int Cg, int dtype, std::initializer_list<const void*> ptrs)
{
    const int eb = elem_bytes(dtype);
    if (eb == 0 || M < 0 || G < 1 || Cg < 1) return DCN_ERR_INVALID_ARG;
    const unsigned long long rows = (unsigned long long)M * (unsigned long long)G;
    if ((long long)Cg * eb >= (1ll << 30) || rows >= (1ull << 40)) return DCN_ERR_UNSUPPORTED;
    gc.rows = rows;
    gc.row_bytes = (uint32_t)(Cg * eb);
    if (M == 0) return DCN_OK;
    for (const void* p : ptrs) {
        if (!p || !aligned(p, (uintptr_t)eb)) return DCN_ERR_INVALID_ARG;
    }
    gc.vb = gc.row_bytes % 16 == 0 ? 16 : eb;
    if ((gc.rows + kGateBlock - 1) / kGateBlock >= (1ull << 31)) return DCN_ERR_UNSUPPORTED;
    gc.blocks = (unsigned)((gc.rows + kGateBlock - 1) / kGateBlock);
    return DCN_OK;
}

template <typename T>
int gate_forward_typed(const GateCall& gc, const void* y, const void* v, const void* z, void* out, bool vec,
                       hipStream_t st)
{
    if (vec)
        hipLaunchKernelGGL((dcn_gate_forward_kernel<T, 16>), dim3(gc.blocks), dim3(kGateBlock), 0, st,
                           (const char*)y, (const char*)v, (const char*)z, (char*)out, gc.rows, gc.row_bytes);
    else
        hipLaunchKernelGGL((dcn_gate_forward_kernel<T, Elem<T>::bytes>), dim3(gc.blocks), dim3(kGateBlock), 0, st,
                           (const char*)y, (const char*)v, (const char*)z, (char*)out, gc.rows, gc.row_bytes);
    return launch_status();
}

template <typename T>
int gate_backward_typed(const GateCall& gc, const void* y, const void* v, const void* z, const void* go, void* gy,
                        void* gv, void* gz, bool vec, hipStream_t st)
{
    if (vec)
        hipLaunchKernelGGL((dcn_gate_backward_kernel<T, 16>), dim3(gc.blocks), dim3(kGateBlock), 0, st,
                           (const char*)y, (const char*)v, (const char*)z, (const char*)go, (char*)gy, (char*)gv,
                           (char*)gz, gc.rows, gc.row_bytes);
    else
        hipLaunchKernelGGL((dcn_gate_backward_kernel<T, Elem<T>::bytes>), dim3(gc.blocks), dim3(kGateBlock), 0, st,
                           (const char*)y, (const char*)v, (const char*)z, (const char*)go, (char*)gy, (char*)gv,
                           (char*)gz, gc.rows, gc.row_bytes);
    return launch_status();
}

}  // namespace

extern "C" int dcn_center_gate_forward(const void* y, const void* v, const void* z, void* output, long long M,
                                       int G, int Cg, int dtype, void* stream)
{
    GateCall gc{};
    int rc = gate_validate(gc, M, G, Cg, dtype, {y, v, z, output});
    if (rc != DCN_OK || M == 0) return rc;
    const bool vec = gc.vb == 16 && aligned(y, 16) && aligned(v, 16) && aligned(output, 16);
    hipStream_t st = (hipStream_t)stream;
    switch (dtype) {
    case DCN_F32: return gate_forward_typed<float>(gc, y, v, z, output, vec, st);
    case DCN_F16: return gate_forward_typed<_Float16>(gc, y, v, z, output, vec, st);
    default: return gate_forward_typed<__bf16>(gc, y, v, z, output, vec, st);
    }
}

extern "C" int dcn_center_gate_backward(const void* y, const void* v, const void* z, const void* grad_output,
                                        void* grad_y, void* grad_v, void* grad_z, long long M, int G, int Cg,
                                        int dtype, void* stream)
{
    GateCall gc{};
    int rc = gate_validate(gc, M, G, Cg, dtype, {y, v, z, grad_output, grad_y, grad_v, grad_z});
    if (rc != DCN_OK || M == 0) return rc;
    const bool vec = gc.vb == 16 && aligned(y, 16) && aligned(v, 16) && aligned(grad_output, 16) &&
                     aligned(grad_y, 16) && aligned(grad_v, 16);
    hipStream_t st = (hipStream_t)stream;
    switch (dtype) {
    case DCN_F32: return gate_backward_typed<float>(gc, y, v, z, grad_output, grad_y, grad_v, grad_z, vec, st);
    case DCN_F16: return gate_backward_typed<_Float16>(gc, y, v, z, grad_output, grad_y, grad_v, grad_z, vec, st);
    default: return gate_backward_typed<__bf16>(gc, y, v, z, grad_output, grad_y, grad_v, grad_z, vec, st);
    }
}

// ---------------------------------------------------------------------------
// Projections of the DCNv4 layer: Y = X W^T + b (dcn_linear.hpp).
#ifndef DCN_LIN_BLOCKS
#define DCN_LIN_BLOCKS 1024
#endif
extern "C" int dcn_linear_forward(const void* x, const void* w, const void* bias, void* y, long long M, int N,
                                  int K, int dtype, void* stream)
{
    const int eb = elem_bytes(dtype);
    if (eb == 0 || M < 0 || N < 1 || K < 1) return DCN_ERR_INVALID_ARG;
    if (M == 0) return DCN_OK;
    if (!x || !w || !y) return DCN_ERR_INVALID_ARG;
    if (!aligned(x, (uintptr_t)eb) || !aligned(w, (uintptr_t)eb) || !aligned(y, (uintptr_t)eb) ||
        (bias && !aligned(bias, (uintptr_t)eb)))
        return DCN_ERR_INVALID_ARG;
    // four-element row chunks: K a multiple of 4 and 16-byte aligned tensors
    if (K % 4 != 0 || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return DCN_ERR_UNSUPPORTED;
    // 64 rows of w, and for half types one 16 x 68 x buffer per wave
    const uint64_t lds = ((uint64_t)kLinNB * (uint64_t)(K + 4) + (eb == 2 ? 4ull * 16ull * 68ull : 0ull)) * (uint64_t)eb;
    const uint64_t m_tiles = ((uint64_t)M + 15) / 16;
    if (lds > 160 * 1024 || m_tiles >= (1ull << 32) || (uint64_t)M * (uint64_t)(K > N ? K : N) >= (1ull << 62))
        return DCN_ERR_UNSUPPORTED;
    // about DCN_LIN_BLOCKS blocks of 4 waves in all, over the column blocks
    const uint32_t gy = (uint32_t)((N + kLinNB - 1) / kLinNB);
    uint64_t gx = (m_tiles + 3) / 4;
    const uint64_t cap = (DCN_LIN_BLOCKS + gy - 1) / gy;
    if (gx > cap) gx = cap;
    LinArgs a{x, w, bias, y, (uint64_t)M, N, K, (uint32_t)m_tiles};
    hipStream_t st = (hipStream_t)stream;
    const dim3 grid((uint32_t)gx, gy);
    switch (dtype) {
    case DCN_F32:
        hipLaunchKernelGGL(dcn_linear_kernel<float>, grid, dim3(kLinBlock), (uint32_t)lds, st, a);
        break;
    case DCN_F16:
        hipLaunchKernelGGL(dcn_linear_kernel<_Float16>, grid, dim3(kLinBlock), (uint32_t)lds, st, a);
        break;
    default:
        hipLaunchKernelGGL(dcn_linear_kernel<__bf16>, grid, dim3(kLinBlock), (uint32_t)lds, st, a);
        break;
    }
    return launch_status();
}

#ifndef DCN_WG_BLOCKS
#define DCN_WG_BLOCKS 512     // blocks of the weight-gradient kernel over all chunks
#endif

namespace {

struct WgPlan {
    uint64_t rows_per_chunk, nchunks;
    int oblocks, iblocks, part_rows, part_ld;
    uint64_t workspace_bytes;
};

// Chunks of a multiple of 64 rows, about DCN_WG_BLOCKS blocks in all.
bool plan_wgrad(long long M, int O, int I, WgPlan& p)
{
    p.oblocks = (O + kWgOB - 1) / kWgOB;
    p.iblocks = (I + kWgIB - 1) / kWgIB;
    p.part_rows = p.oblocks * kWgOB;
    p.part_ld = p.iblocks * kWgIB + 16;
    const uint64_t per = (uint64_t)p.oblocks * (uint64_t)p.iblocks;
    const uint64_t want = per >= DCN_WG_BLOCKS ? 1 : DCN_WG_BLOCKS / per;
    const uint64_t m = M > 0 ? (uint64_t)M : 1;
    const uint64_t rows = ((m + want - 1) / want + kWgRows - 1) / kWgRows * kWgRows;
    p.rows_per_chunk = rows;
    p.nchunks = (m + rows - 1) / rows;
    p.workspace_bytes = p.nchunks * (uint64_t)p.part_rows * (uint64_t)p.part_ld * 4u;
    return rows < (1ull << 31) && p.nchunks < (1ull << 31) && p.oblocks < 65536 && p.iblocks < 65536;
}

template <typename T, int VG>
void launch_wgrad_x(int vx, dim3 grid, const WgArgs& a, hipStream_t st)
{
    if (vx == 16) hipLaunchKernelGGL((dcn_wgrad_kernel<T, VG, 16>), grid, dim3(kWgBlock), 0, st, a);
    else if (vx == 8) hipLaunchKernelGGL((dcn_wgrad_kernel<T, VG, 8>), grid, dim3(kWgBlock), 0, st, a);
    else hipLaunchKernelGGL((dcn_wgrad_kernel<T, VG, 4>), grid, dim3(kWgBlock), 0, st, a);
}

// vg, vx: staging read widths of g and x (16, 8 or 4), both 0 for element reads
template <typename T>
void launch_wgrad(int vg, int vx, dim3 grid, const WgArgs& a, hipStream_t st)
{
    if (vg == 16) launch_wgrad_x<T, 16>(vx, grid, a, st);
    else if (vg == 8) launch_wgrad_x<T, 8>(vx, grid, a, st);
    else if (vg == 4) launch_wgrad_x<T, 4>(vx, grid, a, st);
    else hipLaunchKernelGGL((dcn_wgrad_kernel<T, 0, 0>), grid, dim3(kWgBlock), 0, st, a);
}

// blocks of the fixed-order reduction: one per kWgRedCols 4-column groups of dw
uint64_t wgrad_reduce_blocks(const WgPlan& p, int O)
{
    const int64_t groups = (int64_t)O * (p.part_ld / 4);
    return (uint64_t)((groups + kWgRedCols - 1) / kWgRedCols);
}

template <typename OutT>
int wgrad_zero(OutT* p, int64_t n, hipStream_t st)
{
    if (n <= 0) return DCN_OK;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(dcn_wgrad_zero<OutT>, dim3((uint32_t)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, p, n);
    return launch_status();
}

template <typename OutT>
int wgrad_finish(const WgPlan& p, const void* workspace, void* dw, void* db, int O, int I, hipStream_t st)
{
    const uint64_t rb = wgrad_reduce_blocks(p, O);
    hipLaunchKernelGGL(dcn_wgrad_reduce<OutT>, dim3((uint32_t)rb), dim3(kWgRedCols * kWgRedGroups), 0, st,
                       (const float*)workspace, (OutT*)dw, (OutT*)db, O, I, p.part_rows, p.part_ld,
                       (uint32_t)p.nchunks);
    return launch_status();
}

}  // namespace

extern "C" long long dcn_linear_weight_grad_workspace_size(long long M, int O, int I)
{
    if (M < 0 || O < 1 || I < 1) return -(long long)DCN_ERR_INVALID_ARG;
    if (M == 0) return 0;
    WgPlan p;
    if (!plan_wgrad(M, O, I, p) || wgrad_reduce_blocks(p, O) >= (1ull << 31)) return -(long long)DCN_ERR_UNSUPPORTED;
    return (long long)p.workspace_bytes;
}

extern "C" int dcn_linear_weight_grad(const void* g, const void* x, void* dw, void* db, long long M, int O, int I,
                                      int dtype, int out_dtype, void* workspace, long long workspace_bytes,
                                      void* stream)
{
    const int eb = elem_bytes(dtype), ob = elem_bytes(out_dtype);
    if (eb == 0 || ob == 0 || M < 0 || O < 1 || I < 1 || workspace_bytes < 0 || !dw) return DCN_ERR_INVALID_ARG;
    if (!aligned(dw, (uintptr_t)ob) || (db && !aligned(db, (uintptr_t)ob))) return DCN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    // staging offsets within 64 rows are 32-bit
    if ((int64_t)O * I >= (1ll << 40) || (int64_t)(O > I ? O : I) * eb * kWgRows >= (1ll << 31))
        return DCN_ERR_UNSUPPORTED;
    if (M == 0) {
        // sums over no rows
        int rc = DCN_OK;
        switch (out_dtype) {
        case DCN_F32:
            rc = zero_fill((float*)dw, (int64_t)O * I, st);
            if (rc == DCN_OK && db) rc = zero_fill((float*)db, O, st);
            break;
        case DCN_F16:
            rc = wgrad_zero((_Float16*)dw, (int64_t)O * I, st);
            if (rc == DCN_OK && db) rc = wgrad_zero((_Float16*)db, O, st);
            break;
        default:
            rc = wgrad_zero((__bf16*)dw, (int64_t)O * I, st);
            if (rc == DCN_OK && db) rc = wgrad_zero((__bf16*)db, O, st);
            break;
        }
        return rc;
    }
    if (!g || !x || !aligned(g, (uintptr_t)eb) || !aligned(x, (uintptr_t)eb)) return DCN_ERR_INVALID_ARG;
    WgPlan p;
    if (!plan_wgrad(M, O, I, p) || wgrad_reduce_blocks(p, O) >= (1ull << 31)) return DCN_ERR_UNSUPPORTED;
    if (!workspace || !aligned(workspace, 16) || (uint64_t)workspace_bytes < p.workspace_bytes)
        return DCN_ERR_INVALID_ARG;
    // widest staging read that divides a row of g and of x and keeps every
    // row start aligned (0: element reads)
    auto vec = [&](const void* ptr, int n) {
        if ((n * eb) % 16 == 0 && aligned(ptr, 16)) return 16;
        if ((n * eb) % 8 == 0 && aligned(ptr, 8)) return 8;
        if ((n * eb) % 4 == 0 && aligned(ptr, 4)) return 4;
        return 0;
    };
    int vg = vec(g, O), vx = vec(x, I);
    if (vg == 0 || vx == 0) vg = vx = 0;
    WgArgs a{g, x, (float*)workspace, (uint64_t)M, O, I, (uint32_t)p.rows_per_chunk, p.part_rows, p.part_ld,
             db ? 1 : 0};
    const dim3 grid((uint32_t)p.nchunks, (uint32_t)p.oblocks, (uint32_t)p.iblocks);
    switch (dtype) {
    case DCN_F32: launch_wgrad<float>(vg, vx, grid, a, st); break;
    case DCN_F16: launch_wgrad<_Float16>(vg, vx, grid, a, st); break;
    default: launch_wgrad<__bf16>(vg, vx, grid, a, st); break;
    }
    int rc = launch_status();
    if (rc != DCN_OK) return rc;
    switch (out_dtype) {
    case DCN_F32: return wgrad_finish<float>(p, workspace, dw, db, O, I, st);
    case DCN_F16: return wgrad_finish<_Float16>(p, workspace, dw, db, O, I, st);
    default: return wgrad_finish<__bf16>(p, workspace, dw, db, O, I, st);
    }
}
