// Unquantised (bf16) grouped matmuls for gfx950: forward, dX and tgmm.
//
//   forward  out[m,:] = x[m,:] . w[g(m)]                (reduce over K)
//   dX       dx[m,:]  = dy[m,:] . w[g(m)]^T             (reduce over N)
//   tgmm     dw[g]    = sum_{m in g} x[m,:]^T dy[m,:]   (reduce over M)
//
// "GEMM Kernel 性能优化十问", Q5: the backward pass stays in bf16; Q4: fwd
// reduces over K while tgmm reduces over M, so the same physical M is an
// output dimension in one and the reduction dimension in the other, and each
// phase gets its own tiling.
//
// All three are C[rows][cols] = sum_r A(row, r) B(r, col) on a 128x128 tile
// per workgroup (4 waves, 2x2, each 64x64 = 4x4 v_mfma_f32_16x16x32_bf16
// blocks), staging 64-deep slices of both operands in LDS per step.  An
// operand whose memory layout is contiguous along the reduction index
// (x and dy in forward/dX, w in dX) is read from LDS with ds_read_b128; one
// that is contiguous along the output index (w in forward; x and dy in tgmm,
// where the reduction index M is the row index) is stored as it sits in
// memory and read transposed with ds_read_b64_tr_b16, the in-LDS transpose of
// gfx950.  tgmm walks the expert's rows 64 at a time, so its reduction tile
// is 64 rows while the forward's is 64 K-columns.
#include "gmm_config.hpp"
#include "gmm_device.hpp"
#include "gmm_launch.hpp"

namespace gmm {

namespace {

constexpr int kT = 128;      // output tile (rows and cols)
constexpr int kR = 64;       // reduction depth per LDS stage
// LDS row pitches, chosen by measurement on gfx950 (bytes per CU per clock,
// 16 waves reading one pattern in a loop):
//  - direct [128][64] tiles: 160-byte rows.  A ds_read_b128 of 16 rows at one
//    16-byte chunk runs at ~205 B/clk with this pitch (as fast as a fully
//    contiguous read), ~120 with 144-byte rows and ~63 with unpadded ones.
//  - transposed [64][128] tiles: 288-byte rows.  The ds_read_b64_tr_b16
//    reads of the lane groups that the LDS serves together must land 32
//    banks apart (see read_tr): ~200 B/clk then, ~115 when they collide.
constexpr int kPadD = 16;    // bf16 padding of a direct [128][64] tile
constexpr int kPadT = 16;    // bf16 padding of a transposed [64][128] tile

enum Mode { kFwd = 0, kDx = 1, kTgmm = 2 };

// Transposed fragment of 32-deep reduction block s: the 8 values of column
// c0 + lr (lr = lane % 16) that lane group lg = lane / 16 feeds to the MFMA,
// from a [r][col] LDS tile via two ds_read_b64_tr_b16.  Within each 16-lane
// group, lane i supplies the address of row r + i/4, columns c0 + 4*(i%4)
// .. +3 and receives column c0 + i of rows r .. r+3.
//  - natural order: group lg takes rows 8lg .. 8lg+7 of the block (two reads
//    4 rows apart).  Groups 0 and 1 (and 2 and 3), which the LDS serves in
//    one pass, then read rows 8 apart, 8 x 288 bytes = a multiple of the
//    256-byte bank period: a 2-way bank conflict.
//  - spread order: group lg takes rows 4lg .. 4lg+3 and 16+4lg .. 16+4lg+3.
//    Groups served together read rows 4 apart, 32 banks apart, conflict
//    free.  The MFMA sums over the 32 reduction slots, so any bijection of
//    block rows onto slots gives the same dot product as long as both
//    operands use it; only a call whose other operand is also read here
//    (tgmm) can use it.
template <bool kSpread>
__device__ __forceinline__ v8bf read_tr(const uint16_t* tile, int stride, int s, int lg, int c0, int lr) {
    const int r = s * 32 + (kSpread ? 4 : 8) * lg;
    const uint16_t* p0 = tile + (r + (lr >> 2)) * stride + c0 + (lr & 3) * 4;
    const uint16_t* p1 = p0 + (kSpread ? 16 : 4) * stride;
    const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GMM_LDS v4bf*)(p0));
    const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GMM_LDS v4bf*)(p1));
    return v8bf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ v8bf read_direct(const uint16_t* tile, int stride, int row, int r0) {
    return *reinterpret_cast<const v8bf*>(tile + row * stride + r0);
}

// One thread's share of a staged slice: 4 x 16-byte chunks, chunk c of
// thread t being chunk c*256 + t of the slice in a layout chosen so that
//  - each load instruction reads whole 128-byte lines (8 or 16 lanes per row)
//  - each 16-lane group of an LDS store hits 16 distinct 16-byte bank groups.
// Loads are always issued from in-bounds addresses (callers clamp the row)
// and never consumed before the slice is written to LDS, so a prefetch stays
// in flight while the MFMAs of the current slice run; rows that must read as
// zero are masked when written to LDS.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Frag4 {
    u32x4 d[4];
};

// Direct [128 rows][64] slice (8 chunks per row, LDS rows of 160 bytes):
// instruction c of wave w covers rows R..R+3 and R+8..R+11 with
// R = 16*((4w+c)/2) + 4*((4w+c)%2); lanes 8q..8q+7 take row
// R + q/2 + 8*(q%2), chunks 0..7 (whole 128-byte row segments per 8 lanes;
// ds_write_b128 runs at the same ~78 B/clk/CU for every pattern measured).
__device__ __forceinline__ int direct_row(int c) {
    const int t = threadIdx.x, combo = (t >> 6) * 4 + c, q = (t & 63) >> 3;
    return 16 * (combo >> 1) + 4 * (combo & 1) + (q >> 1) + 8 * (q & 1);
}
__device__ __forceinline__ int direct_chunk() { return threadIdx.x & 7; }

// Transposed-layout [64 rows][128] slice (16 chunks per row, LDS rows of 288
// bytes): chunk c*256 + t is row (c*256 + t)/16, chunk t%16 (a 16-lane group
// is one row).
__device__ __forceinline__ int trans_row(int c) { return (c * 256 + (int)threadIdx.x) >> 4; }
__device__ __forceinline__ int trans_chunk() { return threadIdx.x & 15; }

__device__ __forceinline__ void put_direct(uint16_t* tile, const Frag4& f) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(tile + direct_row(c) * (kR + kPadD) + direct_chunk() * 8) = f.d[c];
}

// Rows r with !valid(r) are written as zeros.
template <typename Valid>
__device__ __forceinline__ void put_trans(uint16_t* tile, const Frag4& f, Valid valid) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int r = trans_row(c);
        *reinterpret_cast<u32x4*>(tile + r * (kT + kPadT) + trans_chunk() * 8) =
            valid(r) ? f.d[c] : u32x4{0u, 0u, 0u, 0u};
    }
}

// tgmm work placement.  A tgmm workgroup owns one 128 x 128 tile of one
// group's dW and walks all of that group's rows, so its cost is the group's
// size.  Blocks run on XCD b % 8 in the order of b.  By default logical ids
// are remapped so that each XCD takes a contiguous run of groups in index
// order, all T tiles of a group on one XCD (its rows of X and dY then fill
// one L2).  Under a skewed routing (the largest group holding more than four
// times the mean rows, e.g. Zipf-popular experts) that leaves some XCD with
// far more rows than the others (1.4x the mean for the production routing),
// so there
//  - every group's T tiles are spread evenly over the 8 XCDs (XCD x takes
//    tiles x*T/8 .. (x+1)*T/8 - 1: with N/128 column tiles per K tile a
//    contiguous band of K tiles, so each column of X is still read by one
//    XCD), and each XCD carries exactly an eighth of the work;
//  - within an XCD, groups go in decreasing size class (>= 2048, >= 512,
//    >= 128 rows, the rest; index order within a class), an approximation of
//    longest-processing-time-first: each freed slot takes the next block, so
//    long tiles started last would set the finishing time.
// Every workgroup derives the same choice and the same order from
// group_sizes alone (a size class depends only on the group's own size), so
// both mappings are bijections from blocks to (group, tile).
__device__ __forceinline__ int tgmm_size_class(int s) {
    return s >= 2048 ? 0 : (s >= 512 ? 1 : (s >= 128 ? 2 : 3));
}

struct TgmmTile {
    int g, t, row_lo, row_hi;
};

// The r-th group of size class cls (cls < 0: of all groups) in index order
// among one chunk of 64 groups, whose clamped row ranges the caller
// supplies (lane i: group base + i); true when found (r is decremented past
// each chunk).
__device__ __forceinline__ bool tgmm_pick(int base, int G, int lo, int hi, int cls, int& r,
                                          TgmmTile& out) {
    const int lane = lane_id();
    const bool in = base + lane < G && (cls < 0 || tgmm_size_class(hi - lo) == cls);
    const unsigned long long mask = __ballot(in);
    const int n = __popcll(mask);
    if (r < n) {
        const unsigned long long sel = __ballot(in && __popcll(mask & ((1ull << lane) - 1ull)) == r);
        const int src = __ffsll((long long)sel) - 1;
        out.g = base + src;
        out.row_lo = lane_value(lo, src);
        out.row_hi = lane_value(hi, src);
        return true;
    }
    r -= n;
    return false;
}

// One wave; every lane gets the result.  T = tiles per group, L = the
// block's id after the default XCD remap.  A group's rows are its clamped
// range (group_chunk: a negative size reads as 0, rows stop at M).  Up to
// 256 groups the ranges stay in registers (one load and one scan per 64
// groups); beyond, the second pass reads and scans them again.
__device__ inline TgmmTile tgmm_tile(const int32_t* __restrict__ group_sizes, int G, int M, int T,
                                     int L, int placement) {
    const bool inreg = G <= 256;
    int glo[4], ghi[4];
    // pass 1: clamped ranges, class counts and the total
    int cnt0 = 0, cnt1 = 0, cnt2 = 0, carry = 0;
    auto count = [&](int base, int sz) {
        const int c = base + lane_id() < G ? tgmm_size_class(sz) : 4;
        cnt0 += __popcll(__ballot(c == 0));
        cnt1 += __popcll(__ballot(c == 1));
        cnt2 += __popcll(__ballot(c == 2));
    };
    if (inreg) {
        // all four loads issued before the first scan: a chain of dependent
        // load round trips is what this prologue would otherwise wait on
        int raw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[c] = group_size_at(group_sizes, G, 64 * c + lane_id());
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            glo[c] = ghi[c] = 0;
            if (64 * c < G) {
                const GroupChunk ch = group_chunk_of(raw[c], M, carry);
                glo[c] = ch.lo;
                ghi[c] = ch.hi;
                carry = ch.next_carry;
                count(64 * c, ch.hi - ch.lo);
            }
        }
    } else {
        for (int base = 0; base < G; base += 64) {
            const GroupChunk ch = group_chunk(group_sizes, G, M, base, carry);
            carry = ch.next_carry;
            count(base, ch.hi - ch.lo);
        }
    }
    const int tot = min(carry, M);
    // skewed: some group holds more than four times the mean (placement 0);
    // placement 1 / 2 force the contiguous / spread mapping (the host checks
    // that spreading has a multiple of 8 tiles per group)
    const bool skewed = placement == 2 || (placement == 0 && T % kNumXcd == 0 && [&] {
        bool big = false;
        if (inreg) {
#pragma unroll
            for (int c = 0; c < 4; ++c) big = big || (int64_t)(ghi[c] - glo[c]) * G > 4 * (int64_t)tot;
        } else {
            int cr = 0;
            for (int base = 0; base < G; base += 64) {
                const GroupChunk ch = group_chunk(group_sizes, G, M, base, cr);
                cr = ch.next_carry;
                big = big || (int64_t)(ch.hi - ch.lo) * G > 4 * (int64_t)tot;
            }
        }
        return __ballot(big) != 0ull;
    }());
    TgmmTile out;
    out.g = -1;   // stays so only for blocks >= G * T (none are launched)
    out.row_lo = out.row_hi = 0;
    int r, cls = -1;   // cls < 0: index order
    if (skewed) {
        const int tx = T / kNumXcd, i = (int)blockIdx.x / kNumXcd;
        r = i / tx;
        out.t = ((int)blockIdx.x % kNumXcd) * tx + i % tx;
        cls = 0;
        if (r >= cnt0) { r -= cnt0; cls = 1;
            if (r >= cnt1) { r -= cnt1; cls = 2;
                if (r >= cnt2) { r -= cnt2; cls = 3; } } }
    } else {
        r = L / T;
        out.t = L % T;
        if (inreg) {   // group r itself: its rows from the ranges in registers
            const int c = r >> 6, l = r & 63;
            const int lo = c == 0 ? glo[0] : (c == 1 ? glo[1] : (c == 2 ? glo[2] : glo[3]));
            const int hi = c == 0 ? ghi[0] : (c == 1 ? ghi[1] : (c == 2 ? ghi[2] : ghi[3]));
            out.g = r;
            out.row_lo = lane_value(lo, l);
            out.row_hi = lane_value(hi, l);
            return out;
        }
    }
    // pass 2: the group at that position and its rows
    if (inreg) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (64 * c < G && tgmm_pick(64 * c, G, glo[c], ghi[c], cls, r, out)) break;
    } else {
        int cr = 0;
        for (int base = 0; base < G; base += 64) {
            const GroupChunk ch = group_chunk(group_sizes, G, M, base, cr);
            cr = ch.next_carry;
            if (tgmm_pick(base, G, ch.lo, ch.hi, cls, r, out)) break;
        }
    }
    return out;
}

// What one workgroup computes: output rows [lo, hi) of the tile starting at
// row0 (forward / dX: rows of group g; tgmm: a K tile of group g's dW),
// columns c0 .. c0 + TC, reduction range [red_lo, red_hi).
struct TileItem {
    int g, row0, lo, hi, c0, red_lo, red_hi;
};

// The prologue every bf16 kernel shares: block 0 writes the call's device
// status word, wave 0 finds the work item (tgmm: the group and tile of
// tgmm_tile over TR x TC tiles; forward / dX: find_work_item over TR-row
// items, placement 2 starting them at each group's first row, TC columns)
// and the workgroup reads it from s_info.  False when the workgroup has
// nothing more to do: no item, or rows past the last group, which it has
// written as zeros.
template <int MODE, bool OUT_BF16, int TR, int TC, int NTHR>
__device__ __forceinline__ bool tile_item(const int32_t* __restrict__ group_sizes, int M, int K, int N, int G,
                                          void* __restrict__ out, int ntiles_c, int ntiles_r, int nblocks,
                                          int placement, int32_t* __restrict__ status, int* s_info, TileItem& it) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int out_cols = MODE == kDx ? K : N;
    if (wave == 1 && blockIdx.x == 0) {   // the call's device status word
        const int st = group_status(group_sizes, G, M);
        if (lane == 0) status[0] = st;
    }
    if constexpr (MODE == kTgmm) {
        const int L = xcd_remap(blockIdx.x, nblocks);
        if (wave == 0) {
            const TgmmTile tt = tgmm_tile(group_sizes, G, M, ntiles_r * ntiles_c, L, placement);
            if (lane == 0) { s_info[0] = tt.row_lo; s_info[1] = tt.row_hi; s_info[2] = tt.g; s_info[3] = tt.t; }
        }
        __syncthreads();
        it.red_lo = s_info[0];
        it.red_hi = s_info[1];
        it.g = s_info[2];
        if (it.g < 0) return false;
        it.row0 = (s_info[3] / ntiles_c) * TR;   // k tile
        it.c0 = (s_info[3] % ntiles_c) * TC;     // n tile
        it.lo = it.row0;
        it.hi = it.row0 + TR;
        return true;
    } else {
        if (wave == 0) {
            // placement 2: row tiles start at each group's first row.  The
            // (row item, column tile) pairs that exist are dealt evenly over
            // the XCDs, a row item's column tiles on one XCD.
            int col;
            const WorkItem wi = placement == 2
                ? balanced_work_item<true>(group_sizes, G, M, TR, ntiles_c, blockIdx.x, col)
                : balanced_work_item(group_sizes, G, M, TR, ntiles_c, blockIdx.x, col);
            if (lane == 0) {
                s_info[0] = wi.g; s_info[1] = wi.tile; s_info[2] = wi.lo; s_info[3] = wi.hi;
                s_info[4] = col;
            }
        }
        __syncthreads();
        it.g = s_info[0];
        if (it.g < 0) return false;
        it.c0 = s_info[4] * TC;
        it.row0 = s_info[1] < 0 ? s_info[2] : s_info[1] * TR;
        it.lo = s_info[2];
        it.hi = s_info[3];
        it.red_lo = 0;
        it.red_hi = MODE == kFwd ? K : N;
        if (it.g == G) {  // rows past the last group: zeros
            const int rows = it.hi - it.lo;
            for (int e = tid; e < rows * (TC / 8); e += NTHR) {
                const int r = it.lo + e / (TC / 8), c = it.c0 + (e % (TC / 8)) * 8;
                if constexpr (OUT_BF16)
                    store_out(reinterpret_cast<uint16_t*>(out) + (int64_t)r * out_cols + c, make_uint4(0, 0, 0, 0));
                else {
                    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (int64_t)r * out_cols + c);
                    store_out(p, make_float4(0, 0, 0, 0));
                    store_out(p + 1, make_float4(0, 0, 0, 0));
                }
            }
            return false;
        }
        return true;
    }
}

constexpr int kTileElems = (kT * (kR + kPadD) > kR * (kT + kPadT)) ? kT * (kR + kPadD) : kR * (kT + kPadT);

// MINB: the minimum waves per SIMD the register allocation must allow (the
// second launch bound); with one wave per SIMD per workgroup it is also the
// number of workgroups a CU can hold.  3 (at most 168 VGPRs; without the
// bound the forward with bf16 output takes 172) for grids of several rounds,
// where more resident workgroups hide more memory latency; 2 for grids that
// fit the chip at two per CU, where a third resident workgroup only lets the
// dispatcher stack work unevenly (measured: production-shape forward 284 ->
// 264 us with 3; wi forward 40.7 -> 42.2 us).
template <int MODE, bool OUT_BF16, int MINB>
__global__ __launch_bounds__(256, MINB) void bf16_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    int ntiles_c, int ntiles_r, int nblocks, int placement, int32_t* __restrict__ status) {
    constexpr bool A_TR = MODE == kTgmm;
    constexpr bool B_TR = MODE != kDx;
    constexpr bool kSpread = A_TR && B_TR;   // both operands transposed: spread reduction order
    __shared__ __attribute__((aligned(16))) uint16_t sA[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kTileElems];
    __shared__ int s_info[5];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int out_cols = MODE == kDx ? K : N;
    TileItem it;
    if (!tile_item<MODE, OUT_BF16, kT, kT, 256>(group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, nblocks, placement,
                                                status, s_info, it))
        return;
    const int g = it.g, row0 = it.row0, lo = it.lo, hi = it.hi, c0 = it.c0, red_lo = it.red_lo, red_hi = it.red_hi;

    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Global -> registers for reduction range [r0, r0 + 64) of both operands,
    // in the chunk layouts above.  Direct A rows are clamped into the item
    // (their values only reach output rows that are never stored); in tgmm
    // rows past the group's end are clamped to its last row here and zeroed
    // when written to LDS.
    const int lda = MODE == kFwd ? K : N;
    const uint16_t* wg = B + (int64_t)(MODE == kTgmm ? 0 : g) * K * N;
    const int dch = direct_chunk() * 8, tch = trans_chunk() * 8;
    auto fetch = [&](Frag4& fa, Frag4& fb, int r0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (MODE == kTgmm) {
                const int m = min(r0 + trans_row(c), red_hi - 1);
                fa.d[c] = *reinterpret_cast<const u32x4*>(A + (int64_t)m * K + row0 + tch);   // x[m][k0..]
                fb.d[c] = *reinterpret_cast<const u32x4*>(B + (int64_t)m * N + c0 + tch);     // dy[m][n0..]
            } else {
                const int arow = min(max(row0 + direct_row(c), lo), hi - 1);
                fa.d[c] = *reinterpret_cast<const u32x4*>(A + (int64_t)arow * lda + r0 + dch);
                if constexpr (MODE == kFwd)   // w[g][k][n0..n0+128]
                    fb.d[c] = *reinterpret_cast<const u32x4*>(wg + (int64_t)(r0 + trans_row(c)) * N + c0 + tch);
                else                          // w[g][k0+c][n]
                    fb.d[c] = *reinterpret_cast<const u32x4*>(wg + (int64_t)(c0 + direct_row(c)) * N + r0 + dch);
            }
        }
    };

    // Software pipeline: the next slice is fetched into registers while the
    // MFMAs of the current one run; one LDS buffer, two barriers per slice.
    // The MFMA operands are swapped (B fragment first) so that each 16x16
    // block comes out transposed: lane (lr, lg) holds row 16i + lr and the
    // four consecutive columns 16j + 4lg .. +3.
    Frag4 fa, fb;
    if (red_lo < red_hi) fetch(fa, fb, red_lo);
    for (int r0 = red_lo; r0 < red_hi; r0 += kR) {
        auto tvalid = [&](int r) { return MODE != kTgmm || r0 + r < red_hi; };
        if constexpr (A_TR) put_trans(sA, fa, tvalid); else put_direct(sA, fa);
        if constexpr (B_TR) put_trans(sB, fb, tvalid); else put_direct(sB, fb);
        __syncthreads();
        if (r0 + kR < red_hi) fetch(fa, fb, r0 + kR);
#pragma unroll
        for (int s = 0; s < kR / 32; ++s) {
            v8bf af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (A_TR)
                    af[i] = read_tr<kSpread>(sA, kT + kPadT, s, lg, wm * 64 + i * 16, lr);
                else
                    af[i] = read_direct(sA, kR + kPadD, wm * 64 + i * 16 + lr, s * 32 + lg * 8);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (B_TR)
                    bf[j] = read_tr<kSpread>(sB, kT + kPadT, s, lg, wn * 64 + j * 16, lr);
                else
                    bf[j] = read_direct(sB, kR + kPadD, wn * 64 + j * 16 + lr, s * 32 + lg * 8);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- epilogue.  bf16: each wave writes its 64 x 64 block into its own
    //      part of the (now idle) LDS tiles and stores it back row by row,
    //      8 lanes x 16 bytes per 128-byte row segment.  fp32: each lane
    //      stores its four consecutive columns (16 bytes).  Rows outside
    //      [lo, hi) are skipped.
    const int64_t obase = MODE == kTgmm ? (int64_t)g * K * N : 0;
    const int col0 = c0 + wn * 64;
    if constexpr (OUT_BF16) {
        constexpr int kEpiRow = 64 + 8;   // bf16 elements per staged row (144 bytes)
        static_assert(4 * 64 * kEpiRow <= 2 * kTileElems, "epilogue staging fits the LDS tiles");
        uint16_t* ep = (wave < 2 ? sA : sB) + (wave & 1) * 64 * kEpiRow;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint2*>(ep + (16 * i + lr) * kEpiRow + 16 * j + 4 * lg) =
                    make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // this wave's writes before its reads
        const int orow = lane >> 3, ocol = (lane & 7) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * q + orow;
            const uint4 v = *reinterpret_cast<const uint4*>(ep + r * kEpiRow + ocol);
            const int row = row0 + wm * 64 + r;
            if (row >= lo && row < hi)
                store_out(reinterpret_cast<uint16_t*>(out) + obase + (int64_t)row * out_cols + col0 + ocol, v);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + wm * 64 + i * 16 + lr;
            if (row < lo || row >= hi) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + obase + (int64_t)row * out_cols + col0 + 16 * j + 4 * lg) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

// ---------------------------------------------------- DMA-fed 128 x 128 --
// The same three products on the 128 x 128 tile and wave layout as above,
// with the operands moved from global memory to LDS by the load-to-LDS
// instructions of gfx950 (global_load_lds_dwordx4: each lane's 16 bytes land
// at the instruction's LDS base + 16 x lane) into a ring of S stages, each
// holding one RD-deep slice of both operands.  The loads of slice t + S - 1
// are issued as soon as every wave has finished reading the stage they
// overwrite, so S - 1 slices are in flight while slice t is multiplied,
// without any registers held for them; each slice costs one workgroup
// barrier.  RES workgroups share a CU; the slice depth is 64 when RES rings
// of 64-deep stages (32 KB each) fit the 160 KB of LDS, else 32 (16 KB):
//   S x RES:  2 x 2, 3 x 1, 4 x 1 -> 64-deep;  3 x 2, 3 x 3, 4 x 2 -> 32-deep.
// More resident waves hide more of each wave's stalls (the barrier, the LDS
// reads); deeper rings keep more bytes in flight per workgroup.
//
// A load-to-LDS instruction writes 1 KB of contiguous LDS, so the stage rows
// cannot be padded; the bank spread comes from XOR swizzles instead:
//  - direct [128][RD] slices (2 RD-byte rows): the 16-byte chunk c of row R
//    sits at chunk c ^ dkey(R), dkey = R % 8 for 128-byte rows, (R / 2) % 4
//    for 64-byte rows.  A ds_read_b128 of 16 rows at one chunk then reads as
//    fast as the padded 160-byte rows (measured ~203 and ~202 B/clk/CU; with
//    (R / 4) % 4, R % 4 or no swizzle the 64-byte rows read at 117-125).
//  - transposed [RD][128] slices (256-byte rows): the 32-byte chunk k of row
//    r sits at chunk k ^ key(r).  The two lane groups the LDS serves
//    together read 8 rows at one chunk (read_tr's row sets), and key takes 8
//    distinct values on each such set: r % 8 for the spread order, r % 4 +
//    4 (bit 3 of r) for the natural one.
// tgmm's last slice may run past the group's rows: the loads there are
// clamped to its last row, and the fragments' rows past the end are zeroed
// in registers before the MFMAs.

template <int S, int RES, int WM, int WN>
struct DmaShape {
    static constexpr int kTR = 64 * WM;                  // tile rows (the A operand's dimension)
    static constexpr int kTC = 64 * WN;                  // tile columns (the B operand's)
    static constexpr int kWaves = WM * WN;
    static constexpr int kStage64 = (kTR + kTC) * 64 * 2;   // bytes of a 64-deep stage
    static constexpr int kRD = RES * S * kStage64 <= 163840 - 1024 ? 64 : 32;   // slice depth
    static constexpr int kSliceA = kTR * kRD;            // bf16 elements of A's slice
    static constexpr int kSliceB = kTC * kRD;            // of B's
    static constexpr int kStage = kSliceA + kSliceB;
    static constexpr int kInstrA = kSliceA * 2 / 1024 / kWaves;   // load-to-LDS instructions per wave
    static constexpr int kInstrB = kSliceB * 2 / 1024 / kWaves;
    static constexpr int kChunks = kRD / 8;              // 16-byte chunks per direct row
    static constexpr int kRows = 64 / kChunks;           // direct rows per instruction
};

template <bool kSpread>
__device__ __forceinline__ int trans_key(int r) {
    return kSpread ? (r & 7) : ((r & 3) | ((r >> 1) & 4));
}

template <int RD>
__device__ __forceinline__ int direct_key(int R) {
    return RD == 64 ? (R & 7) : ((R >> 1) & 3);
}

// Direct fragment: 8 reduction values at chunk `chunk` of row `row`.
template <int RD>
__device__ __forceinline__ v8bf swz_read_direct(const uint16_t* tile, int row, int chunk) {
    return *reinterpret_cast<const v8bf*>(tile + row * RD + 8 * (chunk ^ direct_key<RD>(row)));
}

// The transposed reads of one operand's slice: fragments i = 0..3 of NB
// 32-deep blocks, two ds_read_b64_tr_b16 each, as read_tr lays them out.
// addr[i] is the LDS byte address of fragment i's first read in block 0;
// the second read sits HALF bytes on (rows +4 natural, +16 spread: the same
// key, so the same swizzled chunk), block 1 BLK bytes on (rows +32).  One
// asm block that waits for its own reads before it ends (the
// ds_read_b64_tr_b16 builtin makes the compiler drain every load-to-LDS load
// in flight before it, which would flatten the ring).
typedef unsigned long long u64;
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
template <int NB, int HALF, int BLK>
__device__ __forceinline__ void tr_slice(v8bf (&f)[2][4], const unsigned (&addr)[4]) {
    if constexpr (NB == 2) {
        u64 o[16];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16\n\t"
            "ds_read_b64_tr_b16 %1, %16 offset:%20\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:%21\n\t"
            "ds_read_b64_tr_b16 %3, %16 offset:%22\n\t"
            "ds_read_b64_tr_b16 %4, %17\n\t"
            "ds_read_b64_tr_b16 %5, %17 offset:%20\n\t"
            "ds_read_b64_tr_b16 %6, %17 offset:%21\n\t"
            "ds_read_b64_tr_b16 %7, %17 offset:%22\n\t"
            "ds_read_b64_tr_b16 %8, %18\n\t"
            "ds_read_b64_tr_b16 %9, %18 offset:%20\n\t"
            "ds_read_b64_tr_b16 %10, %18 offset:%21\n\t"
            "ds_read_b64_tr_b16 %11, %18 offset:%22\n\t"
            "ds_read_b64_tr_b16 %12, %19\n\t"
            "ds_read_b64_tr_b16 %13, %19 offset:%20\n\t"
            "ds_read_b64_tr_b16 %14, %19 offset:%21\n\t"
            "ds_read_b64_tr_b16 %15, %19 offset:%22\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
              "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]),
              "=&v"(o[14]), "=&v"(o[15])
            : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(HALF), "i"(BLK), "i"(BLK + HALF)
            : "memory");
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[0][i] = __builtin_bit_cast(v8bf, u64x2{o[4 * i], o[4 * i + 1]});
            f[1][i] = __builtin_bit_cast(v8bf, u64x2{o[4 * i + 2], o[4 * i + 3]});
        }
    } else {
        u64 o[8];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
            "ds_read_b64_tr_b16 %2, %9\n\t"
            "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
            "ds_read_b64_tr_b16 %4, %10\n\t"
            "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
            "ds_read_b64_tr_b16 %6, %11\n\t"
            "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
              "=&v"(o[7])
            : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(HALF)
            : "memory");
#pragma unroll
        for (int i = 0; i < 4; ++i) f[0][i] = __builtin_bit_cast(v8bf, u64x2{o[2 * i], o[2 * i + 1]});
    }
}

// Both operands' transposed reads of a 32-deep slice (tgmm) in one asm
// block, so the slice waits on the LDS once: fragments i = 0..3 of A at
// aa[i] (second read HALF_A bytes on) and of B at ba[i] (HALF_B on).
template <int HALF_A, int HALF_B>
__device__ __forceinline__ void tr_slice_pair(v8bf (&fa)[4], v8bf (&fb)[4], const unsigned (&aa)[4],
                                              const unsigned (&ba)[4]) {
    u64 o[16];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %2, %17\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %18\n\t"
        "ds_read_b64_tr_b16 %5, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %19\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %20\n\t"
        "ds_read_b64_tr_b16 %9, %20 offset:%25\n\t"
        "ds_read_b64_tr_b16 %10, %21\n\t"
        "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
        "ds_read_b64_tr_b16 %12, %22\n\t"
        "ds_read_b64_tr_b16 %13, %22 offset:%25\n\t"
        "ds_read_b64_tr_b16 %14, %23\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
          "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]),
          "=&v"(o[14]), "=&v"(o[15])
        : "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]), "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]),
          "i"(HALF_A), "i"(HALF_B)
        : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[i] = __builtin_bit_cast(v8bf, u64x2{o[2 * i], o[2 * i + 1]});
        fb[i] = __builtin_bit_cast(v8bf, u64x2{o[8 + 2 * i], o[8 + 2 * i + 1]});
    }
}

// The forward's reads of a 32-deep slice in one asm block (one wait): A's
// four direct fragments (16 bytes at da[i]) and B's transposed ones (at
// ba[i], second read HALF_B bytes on).
template <int HALF_B>
__device__ __forceinline__ void direct_tr_slice(v8bf (&fa)[4], v8bf (&fb)[4], const unsigned (&da)[4],
                                                const unsigned (&ba)[4]) {
    v4i d0, d1, d2, d3;
    u64 o[8];
    asm volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %13\n\t"
        "ds_read_b128 %2, %14\n\t"
        "ds_read_b128 %3, %15\n\t"
        "ds_read_b64_tr_b16 %4, %16\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %6, %17\n\t"
        "ds_read_b64_tr_b16 %7, %17 offset:%20\n\t"
        "ds_read_b64_tr_b16 %8, %18\n\t"
        "ds_read_b64_tr_b16 %9, %18 offset:%20\n\t"
        "ds_read_b64_tr_b16 %10, %19\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%20\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3), "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]),
          "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(da[0]), "v"(da[1]), "v"(da[2]), "v"(da[3]), "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]),
          "i"(HALF_B)
        : "memory");
    fa[0] = __builtin_bit_cast(v8bf, d0);
    fa[1] = __builtin_bit_cast(v8bf, d1);
    fa[2] = __builtin_bit_cast(v8bf, d2);
    fa[3] = __builtin_bit_cast(v8bf, d3);
#pragma unroll
    for (int i = 0; i < 4; ++i) fb[i] = __builtin_bit_cast(v8bf, u64x2{o[2 * i], o[2 * i + 1]});
}

// LDS byte address (relative to the slice) of the first read of the
// transposed fragment at columns c0 .. c0+15 in block 0, for this lane, in
// a slice of PITCH-element rows.
template <bool kSpread, int PITCH>
__device__ __forceinline__ unsigned tr_addr(int lg, int c0, int lr) {
    const int r = (kSpread ? 4 : 8) * lg + (lr >> 2);
    return (unsigned)(2 * (r * PITCH + 16 * ((c0 >> 4) ^ trans_key<kSpread>(r)) + (lr & 3) * 4));
}

// A transposed fragment of block s with the reduction rows at or past
// `valid` zeroed (element e holds row r + e for e < 4 and r1 + e - 4 after,
// as read).
template <bool kSpread>
__device__ __forceinline__ v8bf zero_rows_past(v8bf v, int s, int lg, int valid) {
    const int r = s * 32 + (kSpread ? 4 : 8) * lg;
    const int r1 = r + (kSpread ? 16 : 4);
    u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = (q < 2 ? r : r1) + 2 * (q & 1);
        w[q] &= (row < valid ? 0x0000FFFFu : 0u) | (row + 1 < valid ? 0xFFFF0000u : 0u);
    }
    return __builtin_bit_cast(v8bf, w);
}

// Where a lane's load-to-LDS instruction j of one operand's slice reads
// from, relative to the slice's first reduction index.  The instruction
// fills LDS bytes [1024 j, 1024 (j + 1)) of the slice; lane l's 16 bytes go
// to byte 16 l of that kilobyte.
//  direct (rows of 2 RD bytes): kRows rows per instruction, kChunks lanes
//    per row; lane l writes row kRows j + l / kChunks at chunk position
//    l % kChunks, so it loads chunk (l % kChunks) ^ dkey(row): `row` and
//    the element offset `col` of that chunk within the row.
//  transposed (rows of 2 PITCH bytes): 512 / PITCH rows per instruction,
//    PITCH / 8 lanes per row; lane l writes row (512 / PITCH) j + l / (PITCH
//    / 8) at 32-byte position p = (l % (PITCH / 8)) / 2, half l % 2, so it
//    loads 32-byte chunk p ^ key(row), half l % 2: `row` (a reduction index
//    within the slice) and `col`, the element offset within the tile.
struct DmaLane {
    int row, col;
};
template <int RD, int CHUNKS, int ROWS>
__device__ __forceinline__ DmaLane dma_direct(int j, int lane) {
    const int R = ROWS * j + lane / CHUNKS;
    return DmaLane{R, 8 * ((lane % CHUNKS) ^ direct_key<RD>(R))};
}
template <bool kSpread, int PITCH>
__device__ __forceinline__ DmaLane dma_trans(int j, int lane) {
    constexpr int kLanesPerRow = PITCH / 8;
    const int r = (512 / PITCH) * j + lane / kLanesPerRow;
    const int p = (lane % kLanesPerRow) >> 1;
    return DmaLane{r, 16 * (p ^ trans_key<kSpread>(r)) + 8 * (lane & 1)};
}

// WM x WN waves of 64 x 64: a (64 WM) x (64 WN) tile, 2 x 2, 4 x 2 or
// 2 x 4.  The second launch bound is waves per SIMD: RES workgroups of
// WM WN / 4 waves per SIMD.
template <int MODE, bool OUT_BF16, int S, int RES, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, RES * WM * WN / 4) void bf16_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    int ntiles_c, int ntiles_r, int nblocks, int placement, int32_t* __restrict__ status) {
    using D = DmaShape<S, RES, WM, WN>;
    constexpr int RD = D::kRD, TR = D::kTR, TC = D::kTC, NW = D::kWaves, NB = RD / 32;
    constexpr int NIA = D::kInstrA, NIB = D::kInstrB, kSt = D::kStage;
    static_assert((WM == 2 && WN == 2) || (WM == 4 && WN == 2) || (WM == 2 && WN == 4), "2 x 2, 4 x 2 or 2 x 4 waves");
    static_assert(S >= 2 && S <= 4 && RES >= 1 && RES <= 3, "2 to 4 stages, 1 to 3 workgroups per CU");
    static_assert(RES * S * kSt * 2 <= 163840 - 1024, "the rings of RES workgroups fit the LDS");
    static_assert(NIA >= 1 && NIB >= 1 && NIA * NW * 512 == D::kSliceA && NIB * NW * 512 == D::kSliceB,
                  "whole load-to-LDS instructions per wave");
    constexpr int kEpiRow = 64 + 8;   // bf16 epilogue staging row (144 bytes)
    static_assert(!OUT_BF16 || NW * 64 * kEpiRow <= S * kSt, "epilogue staging fits the ring");
    constexpr bool A_TR = MODE == kTgmm;
    constexpr bool B_TR = MODE != kDx;
    constexpr bool kSpread = A_TR && B_TR;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[S * kSt];
    __shared__ int s_info[5];

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int out_cols = MODE == kDx ? K : N;
    TileItem it;
    if (!tile_item<MODE, OUT_BF16, TR, TC, 64 * NW>(group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, nblocks,
                                                    placement, status, s_info, it))
        return;
    const int g = it.g, row0 = it.row0, lo = it.lo, hi = it.hi, c0 = it.c0, red_lo = it.red_lo, red_hi = it.red_hi;

    // ---- this lane's share of a slice: NIA load-to-LDS instructions of A
    //      and NIB of B per wave, instruction i of wave w being j = N w + i
    //      of its operand (dma_direct / dma_trans)
    const int lda = MODE == kFwd ? K : N;
    const uint16_t* wg = B + (int64_t)(MODE == kTgmm ? 0 : g) * K * N;
    int64_t a_off[NIA], b_off[NIB];   // element offsets of the slice at reduction index 0
    int a_row[NIA], b_row[NIB];       // transposed operands: the slice row each instruction fills
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int j = NIA * wave + i;
        if constexpr (MODE == kTgmm) {
            const DmaLane d = dma_trans<kSpread, TR>(j, lane);
            a_row[i] = d.row;
            a_off[i] = row0 + d.col;                            // x[m][k tile]
        } else {
            const DmaLane d = dma_direct<RD, D::kChunks, D::kRows>(j, lane);
            a_row[i] = 0;
            const int arow = min(max(row0 + d.row, lo), hi - 1);
            a_off[i] = (int64_t)arow * lda + d.col;             // x or dy rows
        }
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        const int j = NIB * wave + i;
        if constexpr (MODE == kDx) {
            const DmaLane d = dma_direct<RD, D::kChunks, D::kRows>(j, lane);
            b_row[i] = 0;
            b_off[i] = (int64_t)(c0 + d.row) * N + d.col;       // w[g][k tile][n]
        } else {
            const DmaLane d = dma_trans<kSpread, TC>(j, lane);
            b_row[i] = d.row;
            b_off[i] = c0 + d.col;                              // w[g][k][n tile] or dy[m][n tile]
        }
    }
    auto issue = [&](int t, int stage) {
        const int r0 = red_lo + t * RD;
        uint16_t* sa = ring + stage * kSt;
        uint16_t* sb = sa + D::kSliceA;
#pragma unroll
        for (int i = 0; i < NIA; ++i) {
            const uint16_t* pa;
            if constexpr (MODE == kTgmm)
                pa = A + (int64_t)min(r0 + a_row[i], red_hi - 1) * K + a_off[i];
            else
                pa = A + a_off[i] + r0;
            __builtin_amdgcn_global_load_lds(pa, (GMM_LDS void*)(sa + (NIA * wave + i) * 512), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NIB; ++i) {
            const uint16_t* pb;
            if constexpr (MODE == kTgmm)
                pb = B + (int64_t)min(r0 + b_row[i], red_hi - 1) * N + b_off[i];
            else if constexpr (MODE == kFwd)
                pb = wg + (int64_t)(r0 + b_row[i]) * N + b_off[i];
            else
                pb = wg + b_off[i] + r0;
            __builtin_amdgcn_global_load_lds(pb, (GMM_LDS void*)(sb + (NIB * wave + i) * 512), 16, 0, 0);
        }
    };

    const int wm = (tid >> 6) / WN, wn = (tid >> 6) % WN;
    const int lr = lane & 15, lg = lane >> 4;
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // transposed fragments' lane addresses within a slice (bytes)
    constexpr int kHalfA = (kSpread ? 16 : 4) * TR * 2, kBlkA = 32 * TR * 2;
    constexpr int kHalfB = (kSpread ? 16 : 4) * TC * 2, kBlkB = 32 * TC * 2;
    const unsigned ring_lds = (unsigned)(uintptr_t)(GMM_LDS uint16_t*)ring;
    unsigned a_tr[4], b_tr[4], a_dir[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_tr[i] = tr_addr<kSpread, TR>(lg, wm * 64 + i * 16, lr);
        b_tr[i] = tr_addr<kSpread, TC>(lg, wn * 64 + i * 16, lr);
        const int row = wm * 64 + i * 16 + lr;   // direct A fragment i of block 0 (swz_read_direct)
        a_dir[i] = (unsigned)(2 * (row * RD + 8 * (lg ^ direct_key<RD>(row))));
    }

    const int nsl = (red_hi - red_lo + RD - 1) / RD;
    // unrolled: with a loop of load-to-LDS issues here the compiler's wait
    // insertion drains every load before each LDS read of the main loop
#pragma unroll
    for (int t = 0; t < S - 1; ++t)
        if (t < nsl) issue(t, t);
    int stage = 0;
    for (int t = 0; t < nsl; ++t) {
        // slice t landed in this wave's share once at most the loads of
        // slices t+1 .. t+S-2 (NIA + NIB per slice) are outstanding; the
        // barrier then covers every wave's share, and every wave's reads of
        // the stage the next issue overwrites (slice t - 1's)
        if (t + S - 2 < nsl) wait_vmem<(NIA + NIB) * (S - 2)>(); else wait_vmem<0>();
        stage_barrier();
        if (t + S - 1 < nsl) issue(t + S - 1, stage == 0 ? S - 1 : stage - 1);
        const uint16_t* ta = ring + stage * kSt;
        const uint16_t* tb = ta + D::kSliceA;
        const unsigned sbase = ring_lds + (unsigned)(stage * kSt * 2);
        v8bf atr[2][4], btr[2][4];
        const unsigned bs = sbase + (unsigned)(D::kSliceA * 2);
        if constexpr (!A_TR && B_TR && NB == 1) {   // forward, 32-deep: one wait for both operands
            const unsigned ad[4] = {sbase + a_dir[0], sbase + a_dir[1], sbase + a_dir[2], sbase + a_dir[3]};
            const unsigned bd[4] = {bs + b_tr[0], bs + b_tr[1], bs + b_tr[2], bs + b_tr[3]};
            direct_tr_slice<kHalfB>(atr[0], btr[0], ad, bd);
        } else if constexpr (A_TR && B_TR && NB == 1) {   // tgmm, 32-deep: one wait for both operands
            const unsigned ad[4] = {sbase + a_tr[0], sbase + a_tr[1], sbase + a_tr[2], sbase + a_tr[3]};
            const unsigned bd[4] = {bs + b_tr[0], bs + b_tr[1], bs + b_tr[2], bs + b_tr[3]};
            tr_slice_pair<kHalfA, kHalfB>(atr[0], btr[0], ad, bd);
        } else {
            if constexpr (A_TR) {
                const unsigned ad[4] = {sbase + a_tr[0], sbase + a_tr[1], sbase + a_tr[2], sbase + a_tr[3]};
                tr_slice<NB, kHalfA, kBlkA>(atr, ad);
            }
            if constexpr (B_TR) {
                const unsigned bd[4] = {bs + b_tr[0], bs + b_tr[1], bs + b_tr[2], bs + b_tr[3]};
                tr_slice<NB, kHalfB, kBlkB>(btr, bd);
            }
        }
        const int valid = red_hi - (red_lo + t * RD);   // tgmm: real rows of this slice
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            v8bf af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (A_TR || (B_TR && NB == 1))   // read above (the forward's fused reads)
                    af[i] = atr[s][i];
                else
                    af[i] = swz_read_direct<RD>(ta, wm * 64 + i * 16 + lr, s * 4 + lg);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (B_TR)
                    bf[j] = btr[s][j];
                else
                    bf[j] = swz_read_direct<RD>(tb, wn * 64 + j * 16 + lr, s * 4 + lg);
            }
            if constexpr (MODE == kTgmm) {
                if (valid < RD) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) af[i] = zero_rows_past<kSpread>(af[i], s, lg, valid);
#pragma unroll
                    for (int j = 0; j < 4; ++j) bf[j] = zero_rows_past<kSpread>(bf[j], s, lg, valid);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        stage = stage == S - 1 ? 0 : stage + 1;
    }
    __syncthreads();   // every load landed (the last wait was vmcnt(0)) and every read done

    // ---- epilogue, as the kernel above, staged in the ring
    const int64_t obase = MODE == kTgmm ? (int64_t)g * K * N : 0;
    const int col0 = c0 + wn * 64;
    if constexpr (OUT_BF16) {
        uint16_t* ep = ring + (tid >> 6) * 64 * kEpiRow;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint2*>(ep + (16 * i + lr) * kEpiRow + 16 * j + 4 * lg) =
                    make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const int orow = lane >> 3, ocol = (lane & 7) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * q + orow;
            const uint4 v = *reinterpret_cast<const uint4*>(ep + r * kEpiRow + ocol);
            const int row = row0 + wm * 64 + r;
            if (row >= lo && row < hi)
                store_out(reinterpret_cast<uint16_t*>(out) + obase + (int64_t)row * out_cols + col0 + ocol, v);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + wm * 64 + i * 16 + lr;
            if (row < lo || row >= hi) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + obase + (int64_t)row * out_cols + col0 + 16 * j + 4 * lg) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

template <int MODE, int S, int RES, int WM, int WN>
hipError_t launch_dma(const void* A, const void* B, const int32_t* group_sizes, int M, int K, int N, int G,
                      void* out, bool out_bf16, int placement, int32_t* status, hipStream_t stream) {
    constexpr int TR = 64 * WM, TC = 64 * WN;
    int ntiles_c, ntiles_r = 0;
    int64_t nblocks;
    if constexpr (MODE == kTgmm) {
        ntiles_r = K / TR;
        ntiles_c = N / TC;
        nblocks = (int64_t)G * ntiles_r * ntiles_c;
    } else {
        ntiles_c = (MODE == kFwd ? N : K) / TC;
        nblocks = max_work_items(M, G, TR) * ntiles_c;
    }
    const uint16_t* a = reinterpret_cast<const uint16_t*>(A);
    const uint16_t* b = reinterpret_cast<const uint16_t*>(B);
    if (out_bf16)
        hipLaunchKernelGGL((bf16_dma_kernel<MODE, true, S, RES, WM, WN>), dim3((unsigned)nblocks), dim3(64 * WM * WN), 0,
                           stream, a, b, group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, placement,
                           status);
    else
        hipLaunchKernelGGL((bf16_dma_kernel<MODE, false, S, RES, WM, WN>), dim3((unsigned)nblocks), dim3(64 * WM * WN), 0,
                           stream, a, b, group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, placement,
                           status);
    return hipGetLastError();
}

// ------------------------------------------------------------ wide tiles --
// The same three products on 256x256 output tiles: 8 waves (2 x 4), each
// owning 128 x 64 (8 x 4 MFMA blocks, 128 fp32 accumulators), one workgroup
// per CU.  Each 64-deep step stages 32 KB of each operand, as the 128 x 128
// tile does, for four times the MFMA work: half the L2 reads and LDS writes
// per FLOP, and a quarter fewer LDS reads (128 x 64 wave tiles).  Rows of
// the forward and dX come in 256-row items that start at each group's first
// row; tgmm's tiles are (256 K) x (256 N) per group.  Needs the tile's
// column count (N forward, K dX, K and N tgmm) to be a multiple of 256.
constexpr int kTW = 256;                      // wide tile (rows and cols)
constexpr int kPadTW = 16;                    // transposed [64][256] rows of 544 bytes: rows
                                              // 4 apart land 32 banks apart, as with 288 bytes
constexpr int kWideDirect = kTW * (kR + kPadD);       // bf16 elements of a direct [256][64] tile
constexpr int kWideTrans = kR * (kTW + kPadTW);       // of a transposed [64][256] tile
constexpr int kWideElems = kWideDirect > kWideTrans ? kWideDirect : kWideTrans;

// Chunks of a 256-row direct or 256-column transposed slice per thread.
template <int NWV>
struct WideSlice {
    static constexpr int kThreads = 64 * NWV;
    static constexpr int kChunks = 2048 / kThreads;   // 16-byte chunks per thread and operand
    // Direct [256][64]: instruction c of wave w covers the rows direct_row
    // gives for combo kChunks*w + c (combos 0..31 tile the 256 rows).
    __device__ static int direct_row(int c) {
        const int t = threadIdx.x, combo = (t >> 6) * kChunks + c, q = (t & 63) >> 3;
        return 16 * (combo >> 1) + 4 * (combo & 1) + (q >> 1) + 8 * (q & 1);
    }
    // Transposed [64][256]: chunk c*kThreads + t is row (c*kThreads + t)/32,
    // chunk t%32 (a 16-lane group writes 256 contiguous bytes).
    __device__ static int trans_row(int c) { return (c * kThreads + (int)threadIdx.x) >> 5; }
    __device__ static int trans_chunk() { return threadIdx.x & 31; }
};

// NWV waves as 2 x NWV/2.  Launched with 8 waves of 128 x 64 (128
// accumulators each, two waves per SIMD).  4 waves of 128 x 128 (256
// accumulators, one wave per SIMD) compile, but the compiler then moves the
// accumulators between VGPRs and AGPRs inside the K loop (over 800 copies),
// so that form is not launched.
template <int MODE, bool OUT_BF16, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void bf16_wide_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    int ntiles_c, int ntiles_r, int nblocks, int placement, int32_t* __restrict__ status) {
    using WS = WideSlice<NWV>;
    constexpr int kThr = WS::kThreads, CH = WS::kChunks;
    constexpr int NJ = 256 / (NWV / 2) / 16;        // 16-column blocks per wave (4 or 8)
    constexpr int WC = 16 * NJ;                     // wave tile columns (64 or 128)
    constexpr bool A_TR = MODE == kTgmm;
    constexpr bool B_TR = MODE != kDx;
    constexpr bool kSpread = A_TR && B_TR;
    constexpr int SA = A_TR ? kTW + kPadTW : kR + kPadD;   // LDS row pitches (elements)
    constexpr int SB = B_TR ? kTW + kPadTW : kR + kPadD;
    __shared__ __attribute__((aligned(16))) uint16_t sA[kWideElems];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kWideElems];
    __shared__ int s_info[5];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int out_cols = MODE == kDx ? K : N;
    TileItem it;
    // forward / dX rows come in items starting at each group's first row
    if (!tile_item<MODE, OUT_BF16, kTW, kTW, kThr>(group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, nblocks,
                                              MODE == kTgmm ? placement : 2, status, s_info, it))
        return;
    const int g = it.g, row0 = it.row0, lo = it.lo, hi = it.hi, c0 = it.c0, red_lo = it.red_lo, red_hi = it.red_hi;

    const int wm = wave / (NWV / 2), wn = wave % (NWV / 2);
    const int lr = lane & 15, lg = lane >> 4;
    v4f acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Global -> registers for reduction range [r0, r0 + 64), as in the
    // 128 x 128 kernel (clamped in-bounds rows; tgmm rows past the group's
    // end zeroed when written to LDS).
    const int lda = MODE == kFwd ? K : N;
    const uint16_t* wg = B + (int64_t)(MODE == kTgmm ? 0 : g) * K * N;
    const int dch = direct_chunk() * 8, tch = WS::trans_chunk() * 8;
    u32x4 fa[CH], fb[CH];
    auto fetch = [&](int r0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if constexpr (MODE == kTgmm) {
                const int m = min(r0 + WS::trans_row(c), red_hi - 1);
                fa[c] = *reinterpret_cast<const u32x4*>(A + (int64_t)m * K + row0 + tch);   // x[m][k0..]
                fb[c] = *reinterpret_cast<const u32x4*>(B + (int64_t)m * N + c0 + tch);     // dy[m][n0..]
            } else {
                const int arow = min(max(row0 + WS::direct_row(c), lo), hi - 1);
                fa[c] = *reinterpret_cast<const u32x4*>(A + (int64_t)arow * lda + r0 + dch);
                if constexpr (MODE == kFwd)   // w[g][k][n0..]
                    fb[c] = *reinterpret_cast<const u32x4*>(wg + (int64_t)(r0 + WS::trans_row(c)) * N + c0 + tch);
                else                          // w[g][k0+c][n]
                    fb[c] = *reinterpret_cast<const u32x4*>(wg + (int64_t)(c0 + WS::direct_row(c)) * N + r0 + dch);
            }
        }
    };
    auto put = [&](uint16_t* tile, const u32x4* f, bool trans, int r0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (trans) {
                const int r = WS::trans_row(c);
                const bool valid = MODE != kTgmm || r0 + r < red_hi;
                *reinterpret_cast<u32x4*>(tile + r * (kTW + kPadTW) + WS::trans_chunk() * 8) =
                    valid ? f[c] : u32x4{0u, 0u, 0u, 0u};
            } else {
                *reinterpret_cast<u32x4*>(tile + WS::direct_row(c) * (kR + kPadD) + direct_chunk() * 8) = f[c];
            }
        }
    };

    if (red_lo < red_hi) fetch(red_lo);
    for (int r0 = red_lo; r0 < red_hi; r0 += kR) {
        put(sA, fa, A_TR, r0);
        put(sB, fb, B_TR, r0);
        __syncthreads();
        if (r0 + kR < red_hi) fetch(r0 + kR);
#pragma unroll
        for (int s = 0; s < kR / 32; ++s) {
            v8bf bf[NJ], af[8];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if constexpr (B_TR)
                    bf[j] = read_tr<kSpread>(sB, SB, s, lg, wn * WC + j * 16, lr);
                else
                    bf[j] = read_direct(sB, SB, wn * WC + j * 16 + lr, s * 32 + lg * 8);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (A_TR)
                    af[i] = read_tr<kSpread>(sA, SA, s, lg, wm * 128 + i * 16, lr);
                else
                    af[i] = read_direct(sA, SA, wm * 128 + i * 16 + lr, s * 32 + lg * 8);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- epilogue.  Lane (lr, lg) of block (i, j) holds row 16i + lr and
    //      columns 16j + 4lg .. +3 of the wave's 128 x WC block.  bf16:
    //      staged through LDS by RW waves at a time (128 rows of WC + 8
    //      elements each) and stored as whole rows; fp32: one 16-byte store
    //      per lane and block.  Rows outside [lo, hi) skipped.
    const int64_t obase = MODE == kTgmm ? (int64_t)g * K * N : 0;
    const int col0 = c0 + wn * WC;
    if constexpr (OUT_BF16) {
        constexpr int kEpiRow = WC + 8;
        constexpr int RW = NWV == 8 ? 4 : 2;             // waves staging per round
        static_assert((RW / 2) * 128 * kEpiRow <= kWideElems, "a round's staging fits the LDS tiles");
        constexpr int LPR = WC * 2 / 16;                 // lanes per staged row on the way out
        constexpr int RPP = 64 / LPR;                    // rows per pass
#pragma unroll
        for (int round = 0; round < NWV / RW; ++round) {
            if (wave / RW == round) {
                const int r = wave % RW;
                uint16_t* ep = (r < RW / 2 ? sA : sB) + (r % (RW / 2)) * 128 * kEpiRow;
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        *reinterpret_cast<uint2*>(ep + (16 * i + lr) * kEpiRow + 16 * j + 4 * lg) =
                            make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                const int orow = lane / LPR, ocol = (lane % LPR) * 8;
#pragma unroll
                for (int q = 0; q < 128 / RPP; ++q) {
                    const int rr = RPP * q + orow;
                    const uint4 v = *reinterpret_cast<const uint4*>(ep + rr * kEpiRow + ocol);
                    const int row = row0 + wm * 128 + rr;
                    if (row >= lo && row < hi)
                        store_out(reinterpret_cast<uint16_t*>(out) + obase + (int64_t)row * out_cols + col0 + ocol, v);
                }
            }
            if (round + 1 < NWV / RW) __syncthreads();   // this round's staging read before reuse
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = row0 + wm * 128 + i * 16 + lr;
            if (row < lo || row >= hi) continue;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + obase + (int64_t)row * out_cols + col0 + 16 * j + 4 * lg) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

template <int MODE, int NWV>
hipError_t launch_wide(const void* A, const void* B, const int32_t* group_sizes, int M, int K, int N, int G,
                       void* out, bool out_bf16, int placement, int32_t* status, hipStream_t stream) {
    int ntiles_c, ntiles_r = 0;
    int64_t nblocks;
    if constexpr (MODE == kTgmm) {
        ntiles_r = K / kTW;
        ntiles_c = N / kTW;
        nblocks = (int64_t)G * ntiles_r * ntiles_c;
    } else {
        ntiles_c = (MODE == kFwd ? N : K) / kTW;
        nblocks = max_work_items(M, G, kTW) * ntiles_c;
    }
    const uint16_t* a = reinterpret_cast<const uint16_t*>(A);
    const uint16_t* b = reinterpret_cast<const uint16_t*>(B);
    if (out_bf16)
        hipLaunchKernelGGL((bf16_wide_kernel<MODE, true, NWV>), dim3((unsigned)nblocks), dim3(64 * NWV), 0, stream,
                           a, b, group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, placement, status);
    else
        hipLaunchKernelGGL((bf16_wide_kernel<MODE, false, NWV>), dim3((unsigned)nblocks), dim3(64 * NWV), 0, stream,
                           a, b, group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, placement, status);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const TileConfig& cfg, const void* A, const void* B,
                       const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                       bool out_bf16, int32_t* status, hipStream_t stream) {
    if (cfg.kernel == 2)
        return launch_wide<MODE, 8>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
    if (cfg.kernel == 3) {   // (waves, depth, residency) as gmm_config.cpp accepts them
        const int d = cfg.depth, r = cfg.residency;
        if (cfg.waves == 8 && cfg.tile_n == 256)
            return launch_dma<MODE, 3, 2, 2, 4>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        if (cfg.waves == 8) return launch_dma<MODE, 3, 2, 4, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        if (d == 2) return launch_dma<MODE, 2, 2, 2, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        if (d == 3 && r == 1) return launch_dma<MODE, 3, 1, 2, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        if (d == 3 && r == 2) return launch_dma<MODE, 3, 2, 2, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        if (d == 3) return launch_dma<MODE, 3, 3, 2, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        if (r == 1) return launch_dma<MODE, 4, 1, 2, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
        return launch_dma<MODE, 4, 2, 2, 2>(A, B, group_sizes, M, K, N, G, out, out_bf16, cfg.placement, status, stream);
    }
    int ntiles_c, ntiles_r = 0;
    int64_t nblocks;
    if constexpr (MODE == kTgmm) {
        ntiles_r = K / kT;
        ntiles_c = N / kT;
        nblocks = (int64_t)G * ntiles_r * ntiles_c;
    } else {
        ntiles_c = (MODE == kFwd ? N : K) / kT;
        nblocks = max_work_items(M, G, kT) * ntiles_c;
    }
    const uint16_t* a = reinterpret_cast<const uint16_t*>(A);
    const uint16_t* b = reinterpret_cast<const uint16_t*>(B);
    const dim3 grid((unsigned)nblocks), block(256);
    const int pl = cfg.placement;
    // residency: workgroups per CU the register allocation allows (gmm_config.cpp)
    if (cfg.residency == 2) {
        if (out_bf16)
            hipLaunchKernelGGL((bf16_gemm_kernel<MODE, true, 2>), grid, block, 0, stream, a, b,
                               group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, pl, status);
        else
            hipLaunchKernelGGL((bf16_gemm_kernel<MODE, false, 2>), grid, block, 0, stream, a, b,
                               group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, pl, status);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((bf16_gemm_kernel<MODE, true, 3>), grid, block, 0, stream, a, b,
                               group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, pl, status);
        else
            hipLaunchKernelGGL((bf16_gemm_kernel<MODE, false, 3>), grid, block, 0, stream, a, b,
                               group_sizes, M, K, N, G, out, ntiles_c, ntiles_r, (int)nblocks, pl, status);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_fwd(const TileConfig& cfg, const void* lhs, const void* rhs, const int32_t* group_sizes, int M,
                           int K, int N, int G, void* out, bool out_bf16, int32_t* status, hipStream_t stream) {
    return launch_mode<kFwd>(cfg, lhs, rhs, group_sizes, M, K, N, G, out, out_bf16, status, stream);
}

hipError_t launch_bf16_dx(const TileConfig& cfg, const void* dy, const void* w, const int32_t* group_sizes, int M,
                          int K, int N, int G, void* dx, bool out_bf16, int32_t* status, hipStream_t stream) {
    return launch_mode<kDx>(cfg, dy, w, group_sizes, M, K, N, G, dx, out_bf16, status, stream);
}

hipError_t launch_tgmm(const TileConfig& cfg, const void* x, const void* dy, const int32_t* group_sizes, int M, int K,
                       int N, int G, void* dw, bool out_bf16, int32_t* status, hipStream_t stream) {
    return launch_mode<kTgmm>(cfg, x, dy, group_sizes, M, K, N, G, dw, out_bf16, status, stream);
}

}  // namespace gmm
