// Tile configurations: the library's choice per operation and shape, and the
// process-wide override a tile search sets through gmm_set_tile_config.
#include <mutex>

#include "gmm_config.hpp"
#include "gmm_launch.hpp"

namespace gmm {

namespace {

std::mutex g_mu;
TileConfig g_override[kNumOps] = {};

int64_t items(int64_t M, int64_t G, int64_t tm) { return (M + tm - 1) / tm + G + 1; }

// the row-resident FP8 kernel addresses one expert's weights with 32-bit offsets
bool offsets_fit(int64_t K, int64_t N) { return N * K < (int64_t(1) << 32); }

bool fail(const char** why, const char* w) {
    if (why) *why = w;
    return false;
}

bool any_set(const TileConfig& f) {
    return f.kernel || f.waves || f.tile_m || f.tile_n || f.depth || f.residency || f.placement;
}

// Row-resident sweep: 512-column tiles hold up to 8 K steps in LDS, 256-column
// tiles (bf16 output only) up to 16.
bool rr_fits(int64_t K, int64_t N, int tn, bool out_bf16, bool write_q) {
    if (write_q || !offsets_fit(K, N) || N % tn != 0) return false;
    return tn == 512 ? K <= 1024 : (tn == 256 && K <= 2048 && out_bf16);
}

// FP8 warp-specialised kernel: 1 consecutive items per XCD, 2 each group's
// items on one XCD (one column tile, G within one 64-lane scan).  The
// library takes 2 when the LHS is quantised in the kernel (wi shape: 18.49
// -> 18.25 us, no group's weights fetched into two L2s) and 1 for LHS codes
// (17.30 -> 17.6 us: the busiest XCD gets one item more).
bool group_aligned_fits(int64_t N, int64_t G) { return N == 512 && G <= 64; }

bool resolve_fp8(const TileConfig& f, int64_t M, int64_t K, int64_t N, int64_t G, int lhs_kind,
                 bool out_bf16, bool write_q, TileConfig* c, const char** why) {
    *c = TileConfig{};
    if (!any_set(f)) {   // the library's own choice
        if (N % 512 == 0 && N >= 1024 && rr_fits(K, N, 512, out_bf16, write_q)) {
            c->kernel = kKerRowResident;
            c->tile_m = 48;
            c->tile_n = 512;
            return true;
        }
        c->tile_n = N % 512 == 0 ? 512 : (N % 256 == 0 ? 256 : 128);
        c->tile_m = items(M, G, 48) * (N / c->tile_n) <= device_cus() ? 48 : 64;
        if (c->tile_n == 512 && c->tile_m == 48) {
            c->kernel = kKerWs;
            c->waves = write_q ? 8 : 16;
            c->depth = 1;
            c->placement = lhs_kind != 0 && c->waves == 16 && group_aligned_fits(N, G) ? 2 : 1;
        } else {
            c->kernel = kKerUniform;
        }
        return true;
    }
    if (f.residency) return fail(why, "residency applies to the bf16 calls");
    if (f.placement && f.kernel != kKerWs) return fail(why, "placement applies to the warp-specialised kernel");
    switch (f.kernel) {
        case kKerWs:
            if (N % 512 != 0) return fail(why, "the warp-specialised kernel needs N % 512 == 0");
            if ((f.tile_n && f.tile_n != 512) || (f.tile_m && f.tile_m != 48))
                return fail(why, "the warp-specialised kernel has 48 x 512 tiles");
            c->kernel = kKerWs;
            c->tile_m = 48;
            c->tile_n = 512;
            if (f.waves && f.waves != 8 && f.waves != 12 && f.waves != 16)
                return fail(why, "the warp-specialised kernel runs 8, 12 or 16 waves");
            if (f.depth && f.depth != 1 && f.depth != 2) return fail(why, "depth (weight steps in flight) is 1 or 2");
            c->waves = f.waves ? f.waves : (write_q ? 8 : 16);
            c->depth = f.depth ? f.depth : 1;
            if (write_q && c->waves != 8) return fail(why, "writing the LHS codes takes the 8-wave form");
            if (c->depth == 2 && c->waves != 12) return fail(why, "two steps of weights in flight need 12 waves");
            c->placement = f.placement ? f.placement : 1;
            if (c->placement == 2 && !(c->waves == 16 && group_aligned_fits(N, G)))
                return fail(why, "group-aligned placement needs 16 waves, N == 512 and G <= 64");
            return true;
        case kKerUniform:
            if (f.waves || f.depth) return fail(why, "waves/depth apply to the warp-specialised kernel");
            c->kernel = kKerUniform;
            c->tile_n = f.tile_n ? f.tile_n : (N % 512 == 0 ? 512 : (N % 256 == 0 ? 256 : 128));
            if (N % c->tile_n != 0) return fail(why, "tile_n must divide N");
            if (c->tile_n != 128 && c->tile_n != 256 && c->tile_n != 512)
                return fail(why, "tile_n is 128, 256 or 512");
            c->tile_m = f.tile_m ? f.tile_m
                                 : (items(M, G, 48) * (N / c->tile_n) <= device_cus() ? 48 : 64);
            if (c->tile_m != 48 && c->tile_m != 64) return fail(why, "tile_m is 48 or 64");
            return true;
        case kKerRowResident:
            if (f.waves || f.depth || (f.tile_m && f.tile_m != 48))
                return fail(why, "the row-resident kernel has 48-row tiles of 16 waves");
            c->kernel = kKerRowResident;
            c->tile_m = 48;
            c->tile_n = f.tile_n ? f.tile_n : (K <= 1024 ? 512 : 256);
            if (!rr_fits(K, N, c->tile_n, out_bf16, write_q))
                return fail(why, "the row-resident kernel does not fit this shape (K, N, output dtype or code output)");
            return true;
        default:
            return fail(why, "an FP8 override names its kernel (1, 2 or 3)");
    }
}

bool resolve_mxfp4(const TileConfig& f, int64_t K, int64_t N, TileConfig* c, const char** why) {
    *c = TileConfig{};
    if (!any_set(f)) {
        if (N % 512 == 0 && N >= 1024 && K <= 1024 && offsets_fit(K, N)) {
            c->kernel = kKerRowResident;
            c->tile_n = 512;
        } else {
            c->kernel = kKerWs;
            c->tile_n = N % 512 == 0 ? 512 : (N % 256 == 0 ? 256 : 128);
        }
        c->tile_m = 48;
        c->waves = 16;
        return true;
    }
    if (f.waves && f.waves != 16) return fail(why, "the MXFP4 forward runs 16 waves");
    if ((f.tile_m && f.tile_m != 48) || f.depth || f.residency || f.placement)
        return fail(why, "the MXFP4 forward sets only kernel and tile_n");
    c->tile_m = 48;
    c->waves = 16;
    if (f.kernel == kKerRowResident) {
        c->kernel = kKerRowResident;
        c->tile_n = 512;
        if ((f.tile_n && f.tile_n != 512) || N % 512 != 0 || K > 1024 || !offsets_fit(K, N))
            return fail(why, "the row-resident MXFP4 kernel needs N % 512 == 0 and K <= 1024");
        return true;
    }
    if (f.kernel != kKerWs && f.kernel != kKerAuto) return fail(why, "MXFP4 kernels are 1 or 3");
    c->kernel = kKerWs;
    c->tile_n = f.tile_n ? f.tile_n : (N % 512 == 0 ? 512 : (N % 256 == 0 ? 256 : 128));
    if ((c->tile_n != 128 && c->tile_n != 256 && c->tile_n != 512) || N % c->tile_n != 0)
        return fail(why, "tile_n must be 128, 256 or 512 and divide N");
    return true;
}

// int4 weights: the warp-specialised kernel only (16 waves, 48-row tiles),
// tile_n the widest of 512/256/128 dividing N unless set.
bool resolve_int4(const TileConfig& f, int64_t N, TileConfig* c, const char** why) {
    *c = TileConfig{};
    if ((f.kernel && f.kernel != kKerWs) || (f.waves && f.waves != 16) || (f.tile_m && f.tile_m != 48) ||
        f.depth || f.residency || f.placement)
        return fail(why, "the int4 forward sets only tile_n (warp-specialised, 16 waves, 48 rows)");
    c->kernel = kKerWs;
    c->waves = 16;
    c->tile_m = 48;
    c->tile_n = f.tile_n ? f.tile_n : (N % 512 == 0 ? 512 : (N % 256 == 0 ? 256 : 128));
    if ((c->tile_n != 128 && c->tile_n != 256 && c->tile_n != 512) || N % c->tile_n != 0)
        return fail(why, "tile_n must be 128, 256 or 512 and divide N");
    return true;
}

bool resolve_swiglu(const TileConfig& f, int64_t M, int64_t N, int64_t G, TileConfig* c,
                    const char** why) {
    *c = TileConfig{};
    c->kernel = kKerUniform;
    c->tile_n = 256;
    if (f.tile_m && f.tile_m != 48 && f.tile_m != 64) return fail(why, "tile_m is 48 or 64");
    if ((f.kernel && f.kernel != kKerUniform) || f.waves || (f.tile_n && f.tile_n != 256) || f.depth ||
        f.residency || f.placement)
        return fail(why, "the fused gate+up forward sets only tile_m");
    // 48-row tiles while their grid is at most two rounds of the chip
    c->tile_m = f.tile_m ? f.tile_m : (items(M, G, 48) * (N / 256) <= 2 * device_cus() ? 48 : 64);
    return true;
}

bool resolve_bf16(int op, const TileConfig& f, int64_t M, int64_t K, int64_t N, int64_t G,
                  TileConfig* c, const char** why) {
    *c = TileConfig{};
    if (f.tile_m) return fail(why, "the bf16 calls set kernel, waves, tile_n, residency, depth and placement only");
    if (f.waves && (f.kernel != 3 || (f.waves != 4 && f.waves != 8)))
        return fail(why, "waves (4 or 8) applies to bf16 kernel 3 only");
    if (f.tile_n && (f.waves != 8 || (f.tile_n != 128 && f.tile_n != 256)))
        return fail(why, "tile_n (128 or 256) applies to bf16 kernel 3 with 8 waves");
    if (f.kernel && (f.kernel < 1 || f.kernel > 3))
        return fail(why, "bf16 kernels are 1 (128 x 128), 2 (256 x 256) or 3 (128 x 128 fed by load-to-LDS)");
    if (f.depth && f.kernel && f.kernel != 3) return fail(why, "depth applies to bf16 kernel 3 only");
    if (f.kernel == 2) {
        // 256 x 256 tiles, 8 waves, one workgroup per CU; forward and dX rows
        // in items starting at each group's first row
        const int64_t cols = op == kOpTgmm ? K : (op == kOpDx ? K : N);
        if (cols % 256 != 0 || (op == kOpTgmm && N % 256 != 0))
            return fail(why, "256 x 256 tiles need the tiled dimensions to be multiples of 256");
        if (f.residency && f.residency != 1) return fail(why, "the 256 x 256 kernel runs one workgroup per CU");
        c->kernel = 2;
        c->waves = 8;
        c->residency = 1;
        if (op == kOpTgmm) {
            if (f.placement && f.placement != 1 && f.placement != 2) return fail(why, "placement is 1 or 2");
            if (f.placement == 2 && ((K / 256) * (N / 256)) % 8 != 0)
                return fail(why, "spreading a group over the XCDs needs a multiple of 8 tiles per group");
            c->placement = f.placement;
        } else {
            if (f.placement && f.placement != 2) return fail(why, "the 256 x 256 kernel starts tiles at each group");
            c->placement = 2;
        }
        return true;
    }
    // The library's choice (no kernel, waves, tile_n, depth or residency set;
    // placement may be), from measurements against kernel 1's best on one box:
    //  - tgmm: kernel 3 with 8 waves in 256 x 128 tiles for 128 or more
    //    groups when K is a multiple of 256 (production shape 303 -> 271 us),
    //    else 128 x 128: with few groups a skewed routing leaves the largest
    //    group's tiles on the critical path, and halving their area halves it
    //    (32 groups, Zipf(1.1) routing: 45.6 us with 256 x 128, 37.3 with
    //    128 x 128; uniform routing 29.2 against 28.4);
    //  - forward / dX grids of at most eight 128 x 128 workgroups per CU:
    //    kernel 3, 128 x 128 tiles, 3 stages, three workgroups per CU
    //    (backward shape forward 39.9 -> 33.9 us, dX 37.4 -> 36.1);
    //  - larger forward / dX grids: kernel 3 with 8 waves in 128 x 256 tiles,
    //    which halve the re-reads of the row operand (production shape
    //    forward 257 -> 234 us, dX 273 -> 261); kernel 1 if the tiled
    //    columns are not a multiple of 256.
    // 256-row tiles pad the rows of groups near 256 rows, so the forward and
    // dX never take them by default (backward-shape forward 34 -> 50 us).
    // Set fields: depth implies kernel 3, residency alone kernel 1.
    const int64_t cus = device_cus();
    const int64_t cols = op == kOpDx ? K : N;
    const int64_t nb128 = op == kOpTgmm ? G * (K / 128) * (N / 128) : items(M, G, 128) * (cols / 128);
    int kernel = f.kernel, waves = f.waves, tile_n = f.tile_n;
    if (!f.kernel && !f.waves && !f.tile_n && !f.depth && !f.residency) {
        kernel = 3;
        if (op == kOpTgmm) {
            if (K % 256 == 0 && G >= 128) waves = 8, tile_n = 128;
        } else if (nb128 > 8 * cus) {
            if (cols % 256 == 0)
                waves = 8, tile_n = 256;
            else
                kernel = 1;
        }
    } else if (!kernel) {
        kernel = f.depth ? 3 : 1;
    }
    // kernel 3 with 8 waves: 256 x 128 tiles (tile_n 128; tgmm: 256 K-rows)
    // or 128 x 256 (tile_n 256)
    const int64_t tc = waves == 8 && tile_n == 256 ? 256 : 128;
    const int64_t tr = waves == 8 && tc == 128 ? 256 : 128;
    if (op == kOpTgmm && K % tr != 0) return fail(why, "256 x 128 tgmm tiles need K to be a multiple of 256");
    if (cols % tc != 0) return fail(why, "128 x 256 tiles need the tiled columns to be a multiple of 256");
    const int64_t nblocks = op == kOpTgmm ? G * (K / tr) * (N / tc) : items(M, G, tr) * (cols / tc);
    if (kernel == 3) {
        // LDS stages x workgroups per CU: 64-deep slices (32 KB stages) when
        // the rings fit, else 32-deep (16 KB): 2 x 2, 3 x 1, 4 x 1 (64-deep),
        // 3 x 2, 3 x 3, 4 x 2 (32-deep)
        // 8 waves (256 x 128 tiles): 3 stages of 32-deep slices, 2 per CU
        if (f.depth && (f.depth < 2 || f.depth > 4)) return fail(why, "depth (LDS stages) is 2, 3 or 4");
        c->kernel = 3;
        c->waves = waves ? waves : 4;
        c->tile_n = c->waves == 8 ? (int)tc : 0;
        c->depth = f.depth ? f.depth : 3;
        const int def = c->waves == 8 ? 2 : (c->depth == 2 ? 2 : (c->depth == 3 ? 3 : 2));
        const int res = f.residency ? f.residency : def;
        const bool ok = c->waves == 8 ? c->depth == 3 && res == 2
                                      : (c->depth == 2 ? res == 2 : (c->depth == 3 ? res >= 1 && res <= 3 : res == 1 || res == 2));
        if (!ok)
            return fail(why, "kernel 3 pairs depth 2 with residency 2, 3 with 1-3, 4 with 1-2; with 8 waves depth 3, residency 2");
        c->residency = res;
    } else {
        c->kernel = 1;
        if (f.residency && f.residency != 2 && f.residency != 3) return fail(why, "residency is 2 or 3");
        c->residency = f.residency ? f.residency : (nblocks <= 2 * cus ? 2 : 3);
    }
    if (op == kOpTgmm) {
        if (f.placement && f.placement != 1 && f.placement != 2) return fail(why, "placement is 1 or 2");
        if (f.placement == 2 && ((K / tr) * (N / tc)) % 8 != 0)
            return fail(why, "spreading a group over the XCDs needs a multiple of 8 tiles per group");
        c->placement = f.placement;   // 0: decided in the kernel from the group sizes
    } else {
        // forward and dX: 1 row tiles aligned to absolute rows, 2 row tiles
        // starting at each group's first row.  Group-start tiles leave fewer
        // partly used tiles, which pays once the grid takes more than two
        // rounds of the chip (kernel 1, production shape: dX 284 -> 275 us,
        // forward 264 -> 257 us; kernel 3's 128 x 256 tiles: dX 263 -> 261,
        // forward the same), and for dX at every size since the grid is dealt
        // by the items that exist (backward shape 31.7 -> 28.4 us); the
        // forward's smaller grids keep 1 (backward shape 32.4 against 33.8 us)
        if (f.placement && f.placement != 1 && f.placement != 2) return fail(why, "placement is 1 or 2");
        const bool big = nblocks > 6 * cus && (kernel == 1 || waves == 8);
        c->placement = f.placement ? f.placement : (big || op == kOpDx ? 2 : 1);
    }
    return true;
}

}  // namespace

TileConfig tile_override(int op) {
    std::lock_guard<std::mutex> lock(g_mu);
    return op >= 0 && op < kNumOps ? g_override[op] : TileConfig{};
}

void set_tile_override(int op, const TileConfig* cfg) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_override[op] = cfg ? *cfg : TileConfig{};
}

bool resolve_tile_config(int op, int64_t M, int64_t K, int64_t N, int64_t G, int lhs_kind,
                         bool out_bf16, bool write_q, TileConfig* out, const char** why) {
    const TileConfig f = tile_override(op);
    switch (op) {
        case kOpFp8Fwd: return resolve_fp8(f, M, K, N, G, lhs_kind, out_bf16, write_q, out, why);
        case kOpFp8Swiglu: return resolve_swiglu(f, M, N, G, out, why);
        case kOpFp8Mxfp4: return resolve_mxfp4(f, K, N, out, why);
        case kOpFp8Int4: return resolve_int4(f, N, out, why);
        case kOpBf16Fwd:
        case kOpTgmm:
        case kOpDx: return resolve_bf16(op, f, M, K, N, G, out, why);
        default: *out = TileConfig{}; return true;
    }
}

}  // namespace gmm
