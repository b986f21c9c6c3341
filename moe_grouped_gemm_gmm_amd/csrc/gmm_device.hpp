// Device helpers shared by the gfx950 grouped-matmul kernels: bf16 and FP8
// conversions, the 1x128 quantiser, the in-kernel group metadata routine and
// the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmm {

constexpr int kQBlock = 128;        // quantisation block along K
constexpr float kE4M3Max = 448.0f;  // largest finite OCP E4M3 magnitude
constexpr int kNumXcd = 8;          // MI355X: 8 accelerator complex dies

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

#define GMM_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- bf16 --

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------ quantiser --
// One 1x128 (or 128x128) block: s = a/448 and inv = (s == 0 ? 0 : 1/s), each
// a correctly rounded fp32 division (hipcc's default fp32 divide is IEEE; the
// library is built without fast-math), then code = e4m3_rne(x * inv) with one
// fp32 multiply.  |x*inv| <= 448(1+2^-22) < 464 for every in-contract block,
// and v_cvt_pk_fp8_f32 rounds to nearest even with magnitudes in (448, 464]
// going to 448, so no clamp is needed before the conversion (the GPU tests
// sweep every rounding boundary and compare with the oracle bit for bit).

// s = RN(a / 448).  448 = 7 * 2^6, so a/448 = RN(a/7) * 2^-6 exactly for every
// in-contract a; RN(a/7) is y = RN(a * RN(1/7)) corrected once with the exact
// residual a - 7y (one FMA) and one more FMA.  This equals the IEEE quotient
// for every fp32 significand (checked exhaustively over a binade, which
// covers every exponent since division by 7 commutes with powers of two).
__device__ __forceinline__ float quant_scale7(float a) {   // RN(a / 7)
    constexpr float kInv7 = 0.142857149243354797363281250f;  // RN(1/7)
    const float y = __fmul_rn(a, kInv7);
    const float r = __builtin_fmaf(-y, 7.0f, a);
    return __builtin_fmaf(r, kInv7, y);
}
__device__ __forceinline__ float quant_scale(float a) { return __fmul_rn(quant_scale7(a), 0.015625f); }

// inv = RN(1/s), or 0 when s == 0.  The hardware reciprocal estimate refined
// by one FMA Newton step equals the IEEE quotient 1/s for every significand
// whenever 1/s is a normal number, which holds for every s = a/448 with fp32
// a in the contract (checked exhaustively on gfx950).
__device__ __forceinline__ float quant_inv(float s) {
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, r0, 1.0f);
    const float r1 = __builtin_fmaf(e, r0, r0);
    return s == 0.0f ? 0.0f : r1;
}

// Four fp32 values (already multiplied by inv) -> four E4M3 codes, byte i = value i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    // the first conversion fills bytes 0-1 and keeps the rest of its "old"
    // operand, which the second conversion then overwrites: any register
    // already live will do (here a's bits), so no zero has to be set up
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// int4 weights.  The scale of a 128x128 block is RN(a/7) (quant_scale7; 7 =
// the largest int4 magnitude the quantiser uses) with inverse quant_inv, whose
// reciprocal is normal for every in-contract a, and a code is the weight
// times the inverse rounded half to even, clamped to [-8, 7].
__device__ __forceinline__ int int4_code(float w, float inv) {
    const float y = __builtin_rintf(w * inv);
    return (int)fminf(fmaxf(y, -8.0f), 7.0f);
}

// Four int4 codes (two's complement, one in the low 4 bits of each byte;
// the high bits are ignored) -> their four E4M3 codes, byte for byte.  Every
// integer in [-8, 7] is exact in E4M3: one byte permutation looks up the
// non-negative codes, one the negative ones, and a third picks byte i of
// either result with selector i or 4 + i, the 4 being the nibble's sign bit
// moved to bit 2 of its byte (six instructions per four codes; a blend
// through a 0x00/0xFF mask took seven).
__device__ __forceinline__ uint32_t int4_to_e4m3x4(uint32_t nib) {
    constexpr uint32_t kPos03 = 0x44403800u;   // E4M3 of 0, 1, 2, 3 (bytes 0..3)
    constexpr uint32_t kPos47 = 0x4E4C4A48u;   // 4, 5, 6, 7
    constexpr uint32_t kNeg03 = 0xCACCCED0u;   // -8, -7, -6, -5 (low 3 bits 0..3)
    constexpr uint32_t kNeg47 = 0xB8C0C4C8u;   // -4, -3, -2, -1 (low 3 bits 4..7)
    const uint32_t idx = nib & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(kPos47, kPos03, idx);
    const uint32_t neg = __builtin_amdgcn_perm(kNeg47, kNeg03, idx);
    const uint32_t sel = ((nib >> 1) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(neg, pos, sel);
}

// --------------------------------------------------------- wave helpers --

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// DPP lane permutations (within rows of 16 lanes).
constexpr int kDppXor1 = 0xB1;           // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;           // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;    // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;        // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Lane-group maxima of NON-NEGATIVE floats (abs-max reductions), register
// only.  For x >= 0 the order of the bit patterns as unsigned integers is the
// order of the values, so the reduction runs as unsigned max, whose identity
// 0 lets each DPP move fold into the max instruction.
template <int... CTRLS>
__device__ __forceinline__ float max_nonneg_dpp(float x) {
    uint32_t u = __float_as_uint(x);
    ((u = max(u, dpp<CTRLS>(u))), ...);
    return __uint_as_float(u);
}

// Maximum over each aligned group of 4 lanes (x >= 0).
__device__ __forceinline__ float max_over_4(float x) { return max_nonneg_dpp<kDppXor1, kDppXor2>(x); }

// Maximum over each aligned group of 8 lanes (x >= 0).
__device__ __forceinline__ float max_over_8(float x) {
    return max_nonneg_dpp<kDppXor1, kDppXor2, kDppHalfMirror>(x);
}

// Maximum over each aligned group of 16 lanes (x >= 0).
__device__ __forceinline__ float max_over_16(float x) {
    return max_nonneg_dpp<kDppXor1, kDppXor2, kDppHalfMirror, kDppMirror>(x);
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves only
// (no LDS-crossbar round trips): Hillis-Steele within each row of 16 lanes
// (row_shr 1, 2, 4, 8; lanes shifted in from outside the row read 0), then
// row_bcast:15 adds lane 15's sum (row 0) to row 1 and lane 47's (row 2) to
// row 3, and row_bcast:31 adds lane 31's sum (rows 0-1) to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
    return v;
}

// Value of v in lane `lane`, which must be the same in every lane of the wave.
__device__ __forceinline__ int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Saturating inclusive prefix sum over the 64 lanes: every partial sum is
// min(true sum, cap), for lane values in [0, cap] with cap < 2^31 (then two
// operands add to less than 2^32 and the unsigned sum never wraps; a
// saturating sum of non-negative values is still associative, so the
// Hillis-Steele order of wave_incl_scan gives the same result).
__device__ __forceinline__ uint32_t wave_incl_scan_sat(uint32_t v, uint32_t cap) {
    v = min(v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false), cap);
    v = min(v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false), cap);
    v = min(v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false), cap);
    v = min(v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false), cap);
    v = min(v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false), cap);
    v = min(v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false), cap);
    return v;
}

// The previous lane's value (wave_shr:1); lane 0 gets 0.
__device__ __forceinline__ uint32_t wave_shift_up(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xF, 0xF, false);
}

// ------------------------------------------------------- group metadata --
// Rows of group g are [o_g, o_g + s_g) with o_g = s_0 + ... + s_{g-1}.  The
// kernels only ever touch rows inside [0, M): group_sizes that break the
// contract (a negative size, or sizes summing past M) are read as follows,
// so that no access leaves the caller's buffers:
//  - a negative size counts as 0;
//  - a group's rows are clamped to M: [min(o_g, M), min(o_g + s_g, M)).
// GroupChunk holds, for the 64 groups base .. base+63 (one per lane), the
// clamped row range of the lane's group; `carry` is the clamped row count
// before the chunk (saturated at M + 1, so carry == M + 1 means the sizes so
// far sum past M).
struct GroupChunk {
    int lo, hi;      // clamped rows of group base + lane (lo == hi: empty)
    int next_carry;  // carry for the next chunk
    bool negative;   // some group of the chunk has a negative size
};

// The chunk from the lane's raw size (0 past G), already loaded.
__device__ __forceinline__ GroupChunk group_chunk_of(int raw, int M, int carry) {
    const uint32_t cap = (uint32_t)M + 1u;
    const uint32_t s = (uint32_t)min(max(raw, 0), M + 1);   // cap: a lone group past M still saturates
    const uint32_t incl = wave_incl_scan_sat(s, cap);
    const uint32_t excl = wave_shift_up(incl);
    GroupChunk c;
    c.lo = (int)min(min((uint32_t)carry + excl, cap), (uint32_t)M);
    c.hi = (int)min(min((uint32_t)carry + incl, cap), (uint32_t)M);
    c.next_carry = (int)min((uint32_t)carry + (uint32_t)lane_value((int)incl, 63), cap);
    c.negative = __ballot(raw < 0) != 0ull;
    return c;
}

// group_sizes[g], 0 for g >= G (G >= 1), as an unconditional load of an
// in-bounds index and a select: a conditional load compiles to a branch,
// and the compiler waits for the load at the join, so loads meant to be in
// flight together would each make a round trip of their own.
__device__ __forceinline__ int group_size_at(const int32_t* __restrict__ group_sizes, int G, int g) {
    const int v = group_sizes[min(g, G - 1)];
    return g < G ? v : 0;
}

__device__ __forceinline__ GroupChunk group_chunk(const int32_t* __restrict__ group_sizes, int G,
                                                  int M, int base, int carry) {
    return group_chunk_of(group_size_at(group_sizes, G, base + lane_id()), M, carry);
}

// Bits of the device status word that grouped kernels write (see gmm.h).
constexpr int kDevSumGtM = 1;
constexpr int kDevNegativeSize = 2;

// Device status of group_sizes against M, computed by one wave (every lane
// gets it): kDevSumGtM when the sizes (negative ones read as 0) sum past M,
// kDevNegativeSize when a size is negative.
__device__ __forceinline__ int group_status(const int32_t* __restrict__ group_sizes, int G, int M) {
    int carry = 0, st = 0;
    for (int base = 0; base < G; base += 64) {
        const GroupChunk c = group_chunk(group_sizes, G, M, base, carry);
        carry = c.next_carry;
        if (c.negative) st |= kDevNegativeSize;
    }
    if (carry > M) st |= kDevSumGtM;
    return st;
}

// Work item w of a grouped kernel with row tiles of height tm (a multiple of
// 16), tiles aligned to absolute rows.  Items are ordered group by group;
// each group g with a non-empty clamped row range owns the tiles that
// intersect it, the item's row range being that intersection.  After the
// groups come the items that zero the rows at or past the clamped total
// (g == G).  g < 0 means "no item" (the grid is sized for the worst case:
// at most ceil(M/tm) + G items, since the clamped ranges are disjoint inside
// [0, M)).  Every lane of the calling wave gets the result.  Callers pass a
// compile-time tm, so the divisions become multiply-shifts.

struct WorkItem {
    int g, tile, lo, hi;
};

// GROUP_TILES: tiles start at each group's first row instead (group g's
// rows [o, o + s) give ceil(s / tm) items [o + t tm, min(o + s, o + (t+1) tm)),
// the rows past the total ceil((M - total) / tm) more from `total` on), so
// no item straddles a tile boundary: fewer items with partly used rows
// (about half a tile fewer per group).  `tile` is then -1 and the item's
// rows start at `lo`.  Both mappings give at most max_work_items items.
// Items of a group with clamped rows [lo, hi).
template <bool GROUP_TILES>
__device__ __forceinline__ int group_items(int lo, int hi, int tm) {
    return hi > lo ? (GROUP_TILES ? (hi - lo + tm - 1) / tm : (hi - 1) / tm - lo / tm + 1) : 0;
}

// Items of the rows [total, M) past the clamped total.
template <bool GROUP_TILES>
__device__ __forceinline__ int tail_items(int total, int M, int tm) {
    return total >= M ? 0 : (GROUP_TILES ? (M - total + tm - 1) / tm : (M + tm - 1) / tm - total / tm);
}

// Item w, given that it is the item w - gW of the group g with clamped rows
// [glo, ghi) (GROUP_TILES: tiles from glo; else tiles at multiples of tm).
template <bool GROUP_TILES>
__device__ __forceinline__ WorkItem group_item(int g, int glo, int ghi, int gW, int tm, int w) {
    WorkItem it;
    it.g = g;
    if constexpr (GROUP_TILES) {
        it.tile = -1;
        it.lo = glo + (w - gW) * tm;
        it.hi = min(ghi, it.lo + tm);
    } else {
        const int t = glo / tm + (w - gW);
        it.tile = t;
        it.lo = max(glo, t * tm);
        it.hi = min(ghi, (t + 1) * tm);
    }
    return it;
}

// Tail item w (the items of the groups number items) for the rows past the
// clamped total; g < 0 when it holds no row.
template <bool GROUP_TILES>
__device__ __forceinline__ WorkItem tail_item(int G, int M, int total, int items, int tm, int w) {
    WorkItem it;
    it.g = G;
    if constexpr (GROUP_TILES) {
        it.tile = -1;
        it.lo = total + (w - items) * tm;
        it.hi = min(M, it.lo + tm);
    } else {
        const int t = total / tm + (w - items);
        it.tile = t;
        it.lo = max(total, t * tm);
        it.hi = min(M, (t + 1) * tm);
    }
    if (it.lo >= it.hi) it.g = -1;
    return it;
}

template <bool GROUP_TILES = false>
__device__ __forceinline__ WorkItem find_work_item(const int32_t* __restrict__ group_sizes, int G,
                                                   int M, int tm, int w) {
    int carry_rows = 0, carry_items = 0;
    for (int base = 0; base < G; base += 64) {
        const GroupChunk ch = group_chunk(group_sizes, G, M, base, carry_rows);
        const int c = group_items<GROUP_TILES>(ch.lo, ch.hi, tm);
        const int inclc = wave_incl_scan(c);
        const int W = carry_items + inclc - c;
        const bool own = c > 0 && w >= W && w < W + c;
        const unsigned long long mask = __ballot(own);
        if (mask) {
            const int src = __ffsll((long long)mask) - 1;
            return group_item<GROUP_TILES>(base + src, lane_value(ch.lo, src), lane_value(ch.hi, src),
                                           lane_value(W, src), tm, w);
        }
        carry_rows = ch.next_carry;
        carry_items += lane_value(inclc, 63);
    }
    return tail_item<GROUP_TILES>(G, M, min(carry_rows, M), carry_items, tm, w);
}

// Group-aligned XCD placement of work items, for grids that hold every item
// at once (one workgroup per CU) and one column tile per row tile, G <= 64.
// Blocks run on XCD b % 8; each XCD has `slots` blocks (b / 8 < slots).
// Every group's items go to one XCD (the XCD whose eighth of the item range
// holds the group's midpoint), so a group's weights are fetched into one L2
// only; items (tail items included, after the groups) keep their order
// within an XCD.  An XCD given more items than slots passes the surplus, in
// order, to the spare slots of the XCDs before and after it in XCD order.
// Returns the item index of block b, or -1 (no item).  One wave; every lane
// gets the result.
__device__ __forceinline__ int group_aligned_item(const int32_t* __restrict__ group_sizes, int G,
                                                  int M, int tm, int slots, int b) {
    const int lane = lane_id();
    const GroupChunk ch = group_chunk(group_sizes, G, M, 0, 0);
    const int c = group_items<false>(ch.lo, ch.hi, tm);
    const int inclc = wave_incl_scan(c);
    const int W = inclc - c;                                   // first item of group `lane`
    const int total = min(ch.next_carry, M);
    const int Tg = lane_value(inclc, 63);                      // items of the groups
    const int T = Tg + (total < M ? (M + tm - 1) / tm - total / tm : 0);   // and the tail's
    // XCD of each group: the eighth of [0, T) holding its items' midpoint
    const int xg = T > 0 ? min(7, (8 * (2 * W + c)) / (2 * T)) : 0;
    int start[9];
    start[0] = 0;
    start[8] = T;
#pragma unroll
    for (int x = 1; x < 8; ++x) {
        const unsigned long long m = __ballot(lane < G && c > 0 && xg >= x);
        // no group from x on: XCD x starts where the tail items start
        start[x] = m ? lane_value(W, __ffsll((long long)m) - 1) : Tg;
    }
#pragma unroll
    for (int x = 1; x < 8; ++x) start[x] = max(start[x], start[x - 1]);
    const int x = b % kNumXcd, i = b / kNumXcd;
    const int n = start[x + 1] - start[x];
    if (i < min(n, slots)) return start[x] + i;
    if (n >= slots) return -1;
    // spare slot of XCD x: rank among all spare slots, then the surplus item of that rank
    int rank = i - n;
#pragma unroll
    for (int y = 0; y < 8; ++y)
        if (y < x) rank += max(slots - (start[y + 1] - start[y]), 0);
#pragma unroll
    for (int y = 0; y < 8; ++y) {
        const int extra = max(start[y + 1] - start[y] - slots, 0);
        if (rank < extra) return start[y] + slots + rank;
        rank -= extra;
    }
    return -1;
}

// find_work_item(group_aligned_item(...)) in one pass over group_sizes.  A
// block inside its XCD's own run (every working block unless some XCD has
// more items than slots) needs only the first items of its XCD and the
// next, and the owner of its item is found in the chunk already scanned;
// the other blocks take the full mapping.  The work item, g < 0: none.
__device__ __forceinline__ WorkItem group_aligned_work_item(const int32_t* __restrict__ group_sizes, int G,
                                                           int M, int tm, int slots, int b) {
    const int lane = lane_id();
    const GroupChunk ch = group_chunk(group_sizes, G, M, 0, 0);
    const int c = group_items<false>(ch.lo, ch.hi, tm);
    const int inclc = wave_incl_scan(c);
    const int W = inclc - c;
    const int total = min(ch.next_carry, M);
    const int Tg = lane_value(inclc, 63);
    const int T = Tg + tail_items<false>(total, M, tm);
    const int xg = T > 0 ? min(7, (8 * (2 * W + c)) / (2 * T)) : 0;
    // XCD y's first item: that of its first group (xg is non-decreasing in
    // the group index, so these starts are too), else where the tail starts
    auto first_of = [&](int y) {
        const unsigned long long m = __ballot(lane < G && c > 0 && xg >= y);
        return m ? lane_value(W, __ffsll((long long)m) - 1) : Tg;
    };
    const int x = b % kNumXcd, i = b / kNumXcd;
    const int s0 = x == 0 ? 0 : first_of(x);
    const int s1 = x == kNumXcd - 1 ? T : first_of(x + 1);
    const int w = i < min(s1 - s0, slots) ? s0 + i : group_aligned_item(group_sizes, G, M, tm, slots, b);
    if (w < 0) return WorkItem{-1, 0, 0, 0};
    if (w >= Tg) return tail_item<false>(G, M, total, Tg, tm, w);
    const int src = __ffsll((long long)__ballot(c > 0 && w >= W && w < W + c)) - 1;
    return group_item<false>(src, lane_value(ch.lo, src), lane_value(ch.hi, src), lane_value(W, src), tm, w);
}

// Upper bound of the work-item count for M rows, G groups, tile height tm.
__host__ __device__ inline int64_t max_work_items(int64_t M, int64_t G, int64_t tm) {
    return (M + tm - 1) / tm + G + 1;
}

// Stores of a kernel's results.  Each result line is written once and not
// read again by the kernel that writes it, so the stores carry the
// non-temporal hint: the lines stream out of L2 as they are written instead
// of staying dirty there until the write-back at the end of the kernel,
// which every workgroup would otherwise wait for at once.  Meant for stores
// whose wave covers whole lines; scattered pieces of lines stay plain
// stores, which L2 merges.
__device__ __forceinline__ void store_out(void* p, uint4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, static_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_out(void* p, uint2 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{v.x, v.y}, static_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_out(void* p, float4 v) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, static_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_out(float* p, float v) { __builtin_nontemporal_store(v, p); }

// s_waitcnt vmcnt(N), the other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// A workgroup barrier that leaves the vector memory counter alone (the
// release fence of __syncthreads waits for every load in flight, load-to-LDS
// ones included, which would drain a ring of such loads).  The wavefront fences keep the compiler from moving LDS
// accesses across it; the lgkmcnt wait completes this wave's LDS reads first.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ----------------------------------------------------------- XCD remap --
// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), each with its own L2.  Remap so that consecutive logical ids run on
// the same XCD: neighbours (the N-tiles of one row tile, the row tiles of one
// expert) then share that XCD's L2.  A bijection on [0, nblocks).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
    const int x = bid % kNumXcd, i = bid / kNumXcd;
    const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
    return start + i;
}

// The same contiguous runs, dealt over the `count` logical ids that have
// work instead of the whole grid.  A grid sized for the worst case holds
// more blocks than items; remapping the whole grid would leave its spare
// blocks, and so the idle share, on the last XCDs (at 65536 rows and 256
// groups, 244 of 1538 blocks: one XCD without any work).  XCD x takes
// count / 8 ids (one more for the first count % 8 XCDs) on its first slots;
// returns block bid's id, or -1 for the slots past its XCD's run.  Needs
// count <= nblocks, which max_work_items guarantees for the callers.
__device__ __forceinline__ int xcd_balance(int bid, int count) {
    const int per = count / kNumXcd, rem = count % kNumXcd;
    const int x = bid % kNumXcd, i = bid / kNumXcd;
    if (i >= per + (x < rem ? 1 : 0)) return -1;
    const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
    return start + i;
}

// Number of work items find_work_item<GROUP_TILES> defines for tile height
// tm: every group's items, then the items of the rows past the clamped
// total.  One wave; every lane gets the result.
template <bool GROUP_TILES = false>
__device__ __forceinline__ int work_item_count(const int32_t* __restrict__ group_sizes, int G, int M, int tm) {
    int carry_rows = 0, items = 0;
    for (int base = 0; base < G; base += 64) {
        const GroupChunk ch = group_chunk(group_sizes, G, M, base, carry_rows);
        items += lane_value(wave_incl_scan(group_items<GROUP_TILES>(ch.lo, ch.hi, tm)), 63);
        carry_rows = ch.next_carry;
    }
    return items + tail_items<GROUP_TILES>(min(carry_rows, M), M, tm);
}

// find_work_item<GROUP_TILES> of block b's id under xcd_balance over the
// (item, column tile) pairs that exist, ntiles column tiles per item, in
// one pass over group_sizes: the item (g < 0: none) and, in col, its column
// tile.  Up to 256 groups the clamped ranges and item offsets stay in
// registers, one load per 64 groups, all issued before the first scan (a
// serial chain of dependent loads and scans is what a workgroup's prologue
// waits on); beyond, work_item_count and find_work_item.
template <bool GROUP_TILES = false>
__device__ __forceinline__ WorkItem balanced_work_item(const int32_t* __restrict__ group_sizes, int G, int M,
                                                       int tm, int ntiles, int b, int& col) {
    col = 0;
    if (G > 256) {
        const int L = xcd_balance(b, work_item_count<GROUP_TILES>(group_sizes, G, M, tm) * ntiles);
        if (L < 0) return WorkItem{-1, 0, 0, 0};
        col = L % ntiles;
        return find_work_item<GROUP_TILES>(group_sizes, G, M, tm, L / ntiles);
    }
    const int lane = lane_id();
    int raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = group_size_at(group_sizes, G, 64 * k + lane);
    int lo[4], hi[4], cn[4], W[4];
    int carry = 0, items = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo[k] = hi[k] = cn[k] = W[k] = 0;
        if (64 * k < G) {
            const GroupChunk ch = group_chunk_of(raw[k], M, carry);
            lo[k] = ch.lo;
            hi[k] = ch.hi;
            carry = ch.next_carry;
            cn[k] = group_items<GROUP_TILES>(ch.lo, ch.hi, tm);
            const int incl = wave_incl_scan(cn[k]);
            W[k] = items + incl - cn[k];
            items += lane_value(incl, 63);
        }
    }
    const int total = min(carry, M);
    const int L = xcd_balance(b, (items + tail_items<GROUP_TILES>(total, M, tm)) * ntiles);
    if (L < 0) return WorkItem{-1, 0, 0, 0};
    const int w = L / ntiles;
    col = L % ntiles;
    if (w >= items) return tail_item<GROUP_TILES>(G, M, total, items, tm, w);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned long long m = __ballot(cn[k] > 0 && w >= W[k] && w < W[k] + cn[k]);
        if (m) {
            const int src = __ffsll((long long)m) - 1;
            return group_item<GROUP_TILES>(64 * k + src, lane_value(lo[k], src), lane_value(hi[k], src),
                                           lane_value(W[k], src), tm, w);
        }
    }
    return WorkItem{-1, 0, 0, 0};   // not reached: w < items has an owner
}

}  // namespace gmm
