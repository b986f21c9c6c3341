// Blockwise-FP8 grouped matmul forward for gfx950.
//
// out[m,n] = sum_b ( sum_{k in b} ql[m,k] qr[g,n,k] ) * sl[m,b] * sr[g,b,n/128]
//
// The K loop runs over 128-wide subchannels ("GEMM Kernel 性能优化十问", Q3:
// the K tile is decoupled from the 128-wide quantisation block and every
// subchannel is scaled and accumulated on its own; "实现差距：GMM Kernel
// （V1 vs V2）", section 2.1).  The LHS arrives either as bf16/fp32 and is
// quantised here, per row and subchannel, with the same recipe as
// gmm_quantize_lhs (section 3.3 of the same page), or as E4M3 codes with
// their scales.  The RHS is E4M3 codes with 128x128 block scales, stored by
// gmm_quantize_rhs in the MFMA operand order: per expert, 16-column block and
// subchannel, 2 KB holding the 32 K-values each of the 64 lanes needs as two
// 16-byte runs (byte h*1024 + lane*16 + e is column 16*blk + lane%16,
// k = 128*kb + 32*(lane/16) + 16*h + e).
//
// Work decomposition.  A workgroup of 8 waves (two per SIMD, so one wave's
// VALU work issues while the other's MFMAs run) owns 64 rows of one work item
// (an expert's rows inside a 64-row tile, from the in-kernel metadata
// routine) and TN = 8*WN output columns; wave w owns columns [w*WN, (w+1)*WN)
// of the tile.  Per 128-wide subchannel:
//  - A: wave w quantises rows 8w..8w+7; a lane holds 16 K values of one row
//    (8 lanes per row; each load instruction reads whole 128-byte lines) and
//    the row's abs-max is reduced over those 8 lanes with DPP.  Every row is
//    quantised once per workgroup.  Codes go to a double-buffered LDS tile,
//    and with them the products sl[row] * sr[n-block] for each 128-column
//    block of the tile, so the MFMA waves read their per-row factors
//    ready-made.
//  - B: each wave loads its own columns straight from global memory into the
//    MFMA operand registers: two 16-byte loads per lane per 16-column block,
//    each instruction reading one contiguous kilobyte of the packed RHS.  No
//    two waves share B, so it never goes through LDS.  B is double-buffered
//    in registers: the next subchannel's B is requested at the start of a
//    step, a whole step before its MFMAs.
//  - Raw A (with the RHS scale its lane folds in) is loaded two subchannels
//    ahead and quantised one ahead of the MFMAs that use it; one barrier per
//    subchannel.  The loop body has no branches (prefetch indices are
//    clamped) and issues its loads in the same order every step, so the
//    compiler's waits are counts rather than full drains.
//  - Inside a step each MFMA is followed by a slice of independent VALU work
//    (the next subchannel's quantiser, earlier blocks' scale FMAs), so the
//    VALU and the matrix core run side by side.
//  - Each 16x16 block is one v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0
//    scales: the FP8 products are exact) into a zero temporary, folded into
//    the fp32 accumulator with one FMA per element: acc += p * (sl * sr).
//  - The MFMA operands are swapped so every 16x16 block comes out transposed:
//    a lane owns one output row and four consecutive columns, which makes the
//    row factor one scalar per block and lets the epilogue store 8-byte (bf16)
//    or 16-byte (fp32) runs directly.
#include <algorithm>
#include <type_traits>

#include "gmm_config.hpp"
#include "gmm_device.hpp"
#include "gmm_launch.hpp"

namespace gmm {

namespace {

constexpr int kTK = 128;           // one subchannel
constexpr int kTM = 64;            // rows the quantiser covers (LDS tile height)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsRow = kTK + 16;  // 144-byte LDS rows: conflict-free 16-lane ds_read_b128

enum LhsKind { kLhsE4M3 = 0, kLhsBF16 = 1, kLhsF32 = 2 };

#ifndef GMM_FP8_VALU_PER_MFMA
#define GMM_FP8_VALU_PER_MFMA 8   // VALU instructions scheduled after each MFMA
#endif

// Quantiser geometry: the 64 x 128 subchannel tile is split evenly over the
// 512 lanes, 8 lanes per row, 16 values per lane in two runs of 8; run p of
// lane chunk c holds the K values 8c + 64p .. +7, so each load instruction of a
// wave reads the same 128-byte half of 8 rows.
constexpr int kLPR = 8;                 // lanes per row
constexpr int kRPW = 64 / kLPR;         // rows per wave
constexpr int kNP = 2;                  // runs of 8 values per lane

// Raw LHS registers of one subchannel for this lane.  Lanes of rows outside
// the work item load a clamped in-bounds row; their codes only reach output
// rows that are never stored.
template <int KIND>
struct RawA;
template <>
struct RawA<kLhsBF16> { uint4 d[kNP]; };
template <>
struct RawA<kLhsF32> { uint4 d[2 * kNP]; };
template <>
struct RawA<kLhsE4M3> { uint2 d[kNP]; float s; };

template <int KIND>
__device__ __forceinline__ void load_raw(RawA<KIND>& r, const void* __restrict__ lhs,
                                         const float* __restrict__ lhs_scale, int64_t row, int K,
                                         int kb, int chunk) {
    const int64_t e = row * K + kb * kTK + chunk * 8;
#pragma unroll
    for (int p = 0; p < kNP; ++p) {
        const int64_t ep = e + p * 8 * kLPR;
        if constexpr (KIND == kLhsBF16) {
            r.d[p] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(lhs) + ep);
        } else if constexpr (KIND == kLhsF32) {
            const float* q = reinterpret_cast<const float*>(lhs) + ep;
            r.d[2 * p] = *reinterpret_cast<const uint4*>(q);
            r.d[2 * p + 1] = *reinterpret_cast<const uint4*>(q + 4);
        } else {
            r.d[p] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(lhs) + ep);
        }
    }
    if constexpr (KIND == kLhsE4M3) r.s = lhs_scale[row * (K / kTK) + kb];
}

// 16 values -> 16 codes (two runs of 8) and the row's scale; the abs-max is
// reduced over the 8 lanes that hold the row (DPP, no LDS round trip).
template <int KIND>
__device__ __forceinline__ float quantize_raw(const RawA<KIND>& r, uint2 (&codes)[kNP]) {
    if constexpr (KIND == kLhsE4M3) {
#pragma unroll
        for (int p = 0; p < kNP; ++p) codes[p] = r.d[p];
        return r.s;
    } else {
        float v[8 * kNP];
        if constexpr (KIND == kLhsBF16) {
#pragma unroll
            for (int q = 0; q < kNP; ++q) {
                v[8 * q + 0] = bf16_lo(r.d[q].x); v[8 * q + 1] = bf16_hi(r.d[q].x);
                v[8 * q + 2] = bf16_lo(r.d[q].y); v[8 * q + 3] = bf16_hi(r.d[q].y);
                v[8 * q + 4] = bf16_lo(r.d[q].z); v[8 * q + 5] = bf16_hi(r.d[q].z);
                v[8 * q + 6] = bf16_lo(r.d[q].w); v[8 * q + 7] = bf16_hi(r.d[q].w);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 2 * kNP; ++q) {
                v[4 * q + 0] = __uint_as_float(r.d[q].x); v[4 * q + 1] = __uint_as_float(r.d[q].y);
                v[4 * q + 2] = __uint_as_float(r.d[q].z); v[4 * q + 3] = __uint_as_float(r.d[q].w);
            }
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8 * kNP; ++i) a = fmaxf(a, fabsf(v[i]));
        a = max_over_8(a);
        const float s = quant_scale(a);
        const float inv = quant_inv(s);
#pragma unroll
        for (int q = 0; q < kNP; ++q) {
            codes[q].x = e4m3x4(v[8 * q + 0] * inv, v[8 * q + 1] * inv, v[8 * q + 2] * inv, v[8 * q + 3] * inv);
            codes[q].y = e4m3x4(v[8 * q + 4] * inv, v[8 * q + 5] * inv, v[8 * q + 6] * inv, v[8 * q + 7] * inv);
        }
        return s;
    }
}

template <int WN>
struct Smem {
    static constexpr int TN = kWaves * WN;
    static constexpr int NBLK = TN / 128 > 0 ? TN / 128 : 1;   // 128-column scale blocks per tile
    static_assert(NBLK <= kLPR, "one quantiser lane per 128-column block");
    uint8_t a[2][kTM][kLdsRow];         // E4M3 codes of the current and next subchannel
    float c[2][kLPR][kTM];              // sl[row] * sr[n-block]; one slot per quantiser lane
                                        // (slots >= NBLK are written, never read)
};

// Shared memory of a workgroup: the loop's A tiles, or, after the loop, each
// wave's bf16 output block (64 rows x WN columns, rows padded by 16 bytes) for
// the row-contiguous write-back.
template <int WN>
union SmemAll {
    static constexpr int kEpiRow = WN * 2 + 16;
    Smem<WN> m;
    uint8_t epi[kWaves][kTM][kEpiRow];
};

// What one lane needs to quantise one subchannel: its raw LHS values and the
// RHS scale of the 128-column block whose per-row factor it writes.
template <int KIND>
struct Stage {
    RawA<KIND> raw;
    float sr;
};

// TM (64 or 48) is the row-tile height.  With 48-row tiles the quantiser
// still covers 64 rows: the last 16 lie past the tile, are never valid for the
// item and are never read by an MFMA, so the quantiser and the LDS layout stay
// the same while each workgroup does three quarters of the MFMA work and more
// workgroups share the chip.
//
// SWIGLU: the fused gate+up projection ("实现差距：GMM Kernel（V1 vs V2）",
// sections 3.5 and 4.2).  The RHS has 2N columns, the gate projection in the
// first N and the up projection in the next N; the output is
// silu(gate) * up, N columns.  A workgroup covers 256 output columns: wave w
// owns gate columns n0 + 32w .. +31 (its B blocks 0, 1) and the matching up
// columns N + n0 + 32w .. +31 (blocks 2, 3), so the activation is formed in
// registers.  With act_q non-null the activation is also quantised 1x128
// (same recipe as the LHS) for the next layer: each 128-column block spans
// four waves, whose row maxima meet in LDS.
template <int KIND, bool OUT_BF16, int WN, int TM, bool WRITE_Q, bool SWIGLU>
__global__ __launch_bounds__(kThreads, 2) void fp8_fwd_kernel(
    const void* __restrict__ lhs, const float* __restrict__ lhs_scale,
    const uint8_t* __restrict__ rhs, const float* __restrict__ rhs_scale,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    uint8_t* __restrict__ q_out, float* __restrict__ s_out, int ntiles_n, int nblocks,
    int32_t* __restrict__ status) {
    static_assert(TM == 64 || TM == 48, "64- or 48-row tiles");
    constexpr int MB = TM / 16;   // 16-row blocks of the tile
    constexpr int NB = WN / 16;   // 16-column blocks per wave
    static_assert(!SWIGLU || (WN == 64 && !WRITE_Q), "fused gate+up uses 64-column waves");
    constexpr int TN = SWIGLU ? kWaves * WN / 2 : kWaves * WN;   // output columns per tile
    constexpr int NBLK = Smem<WN>::NBLK;
    constexpr int OUT_BYTES = OUT_BF16 ? 2 : 4;

    __shared__ WorkItem s_item;
    __shared__ __attribute__((aligned(16))) SmemAll<WN> smu;
    __shared__ float s_rmax[SWIGLU ? kWaves : 1][SWIGLU ? kTM : 1];   // activation row maxima
    Smem<WN>& sm = smu.m;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ int s_nt;
    if (wave == 0) {
        // the (row item, column tile) pairs that exist, dealt evenly over the XCDs
        int col;
        const WorkItem it = balanced_work_item(group_sizes, G, M, TM, ntiles_n, blockIdx.x, col);
        if (lane == 0) {
            s_item = it;
            s_nt = col;
        }
    } else if (wave == 1 && blockIdx.x == 0) {   // the call's device status word
        const int st = group_status(group_sizes, G, M);
        if (lane == 0) status[0] = st;
    }
    __syncthreads();
    const WorkItem it = s_item;
    if (it.g < 0) return;
    const int nt = s_nt;
    const int n0 = nt * TN;

    if (it.g == G) {  // rows past the last group: zeros
        const int rows = it.hi - it.lo;
        constexpr int V = 16 / OUT_BYTES;  // elements per 16-byte store
        for (int e = tid; e < rows * (TN / V); e += kThreads) {
            const int r = it.lo + e / (TN / V), c = n0 + (e % (TN / V)) * V;
            store_out(reinterpret_cast<uint8_t*>(out) + ((int64_t)r * N + c) * OUT_BYTES,
                make_uint4(0, 0, 0, 0));
        }
        if (SWIGLU && q_out != nullptr) {   // their activation codes and scales too
            for (int e = tid; e < rows * (TN / 16); e += kThreads) {
                const int r = it.lo + e / (TN / 16), c = n0 + (e % (TN / 16)) * 16;
                store_out(q_out + (int64_t)r * N + c, make_uint4(0, 0, 0, 0));
            }
            for (int e = tid; e < rows * (TN / kQBlock); e += kThreads) {
                const int r = it.lo + e / (TN / kQBlock), b = n0 / kQBlock + e % (TN / kQBlock);
                s_out[(int64_t)r * (N / kQBlock) + b] = 0.0f;
            }
        }
        return;
    }

    const int g = it.g, row0 = it.tile * TM;
    const int NR = SWIGLU ? 2 * N : N;            // RHS columns
    const int nkb = K / kTK, nnb = NR / kQBlock;

    // ---- quantiser role: row 8*wave + lane/8, chunk c = lane % 8
    const int qchunk = lane % kLPR;
    const int qrow = kRPW * wave + lane / kLPR;
    const int64_t qgrow = row0 + qrow;
    const bool qvalid = qgrow >= it.lo && qgrow < it.hi;
    const int64_t qlrow = qvalid ? qgrow : it.lo;    // in-bounds row the loads use
    const bool write_q = WRITE_Q && nt == 0 && qvalid;
    // RHS scale this lane folds into its row factor: 128-column block qchunk
    // of the tile (clamped; lanes past NBLK write an unused slot)
    // (fused gate+up: slots 0, 1 are the tile's gate blocks, 2, 3 its up blocks)
    const int qslot = min(qchunk, NBLK - 1);
    const int qblk = !SWIGLU ? n0 / kQBlock + qslot
                             : (qslot < 2 ? n0 / kQBlock + qslot : (N + n0) / kQBlock + qslot - 2);
    const float* srl = rhs_scale + (int64_t)g * nkb * nnb + qblk;

    // ---- MFMA role: columns [n0 + wave*WN, +WN); lane = row/col lr, K chunk lc.
    //      B is the packed RHS: 2 KB per (16-column block, subchannel), this
    //      lane's 32 codes at byte lane*16 of each 1 KB half.
    const int lr = lane & 15, lc = lane >> 4;
    const int ncol0 = SWIGLU ? n0 + 32 * wave : n0 + wave * WN;    // first output column
    // factor slots of the wave's column blocks (j < NB/2 and j >= NB/2 for
    // the fused projection)
    const int slot_lo = SWIGLU ? wave / 4 : (wave * WN) / 128;
    const int slot_hi = SWIGLU ? 2 + wave / 4 : slot_lo;
    const uint8_t* bptr = rhs + ((int64_t)g * (NR / 16) + ncol0 / 16) * nkb * 2048 + lane * 16;
    // B block j >= NB/2 of the fused projection: the up columns, N further on
    const int64_t bup = SWIGLU ? (int64_t)(N / 16) * nkb * 2048 - (int64_t)(NB / 2) * nkb * 2048 : 0;

    v4f acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto load_stage = [&](Stage<KIND>& st, int kb) {
        load_raw<KIND>(st.raw, lhs, lhs_scale, qlrow, K, kb, qchunk);
        st.sr = srl[kb * nnb];
    };
    // Quantise a stage (subchannel kb) into LDS buffer buf.
    auto quant_store = [&](int kb, int buf, const Stage<KIND>& st) {
        uint2 codes[kNP];
        const float s = quantize_raw<KIND>(st.raw, codes);
#pragma unroll
        for (int p = 0; p < kNP; ++p)
            *reinterpret_cast<uint2*>(&sm.a[buf][qrow][qchunk * 8 + p * 8 * kLPR]) = codes[p];
        sm.c[buf][qchunk][qrow] = s * st.sr;
        if (write_q) {
#pragma unroll
            for (int p = 0; p < kNP; ++p)
                *reinterpret_cast<uint2*>(q_out + qgrow * K + kb * kTK + qchunk * 8 + p * 8 * kLPR) = codes[p];
            if (qchunk == 0) s_out[qgrow * nkb + kb] = s;
        }
    };
    auto load_b = [&](v8i (&b)[NB], int kb) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const uint8_t* p = bptr + ((int64_t)j * nkb + kb) * 2048 + (j >= NB / 2 ? bup : 0);
            const uint4 lo = *reinterpret_cast<const uint4*>(p);
            const uint4 hi = *reinterpret_cast<const uint4*>(p + 1024);
            b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };

    // Step kb.  B of kb+1 is requested first, into the register set the MFMAs
    // of this step do not use; the A fragments of kb are read from LDS; the
    // stage quantised now (kb+1, into the other LDS buffer) was loaded two
    // steps earlier and is reloaded at once with kb+3.  The loads are issued
    // in the same order every step (B, then the stage) and the prologue issues
    // them in that order too, so the waits the compiler places are counts,
    // not full drains.  Indices past the last subchannel are clamped to it
    // (redundant reloads instead of branches).
    auto step = [&](int kb, v8i (&bc)[NB], v8i (&bn)[NB], Stage<KIND>& sq) {
        const int buf = kb & 1;
        const int kb1 = min(kb + 1, nkb - 1), kb3 = min(kb + 3, nkb - 1);
        load_b(bn, kb1);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the quantiser's VALU work
        // Operands are swapped so each 16x16 block comes out transposed: lane
        // (lr, lc) holds row 16i + lr and the four consecutive columns
        // 16j + 4lc .. +3, so its per-row factor sl * sr is one scalar per row
        // block.
        // All A fragments are read up front, except in the code-writing
        // variant, which reads one row block at a time to stay within the
        // register budget.
        constexpr bool kAllA = !WRITE_Q;
        constexpr int NF = SWIGLU ? 2 : 1;      // row factors per row block (gate, up)
        v8i af[kAllA ? MB : 1];
        float cf[kAllA ? MB : 1][NF];
        auto read_cf = [&](float (&c)[NF], int i) {
            c[0] = sm.c[buf][slot_lo][16 * i + lr];
            if constexpr (SWIGLU) c[1] = sm.c[buf][slot_hi][16 * i + lr];
        };
        if constexpr (kAllA) {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                af[i] = *reinterpret_cast<const v8i*>(&sm.a[buf][16 * i + lr][lc * 32]);
                read_cf(cf[i], i);
            }
        }
        quant_store(kb1, buf ^ 1, sq);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int ia = kAllA ? i : 0;
            if constexpr (!kAllA) {
                af[0] = *reinterpret_cast<const v8i*>(&sm.a[buf][16 * i + lr][lc * 32]);
                read_cf(cf[0], i);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bc[j], af[ia], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                const float f = cf[ia][SWIGLU && j >= NB / 2 ? 1 : 0];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], f, acc[i][j][r]);
            }
        }
        load_stage(sq, kb3);
        // Issue order inside the step: the A-fragment reads, then each MFMA
        // followed by a slice of VALU work (the next subchannel's quantiser
        // and earlier blocks' scale FMAs) so that VALU issues while the
        // matrix core runs, then the LDS stores and the stage loads.
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * MB + MB / 2, 0);
#pragma unroll
        for (int q = 0; q < MB * NB; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, GMM_FP8_VALU_PER_MFMA, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
        __syncthreads();
    };

    // ---- prologue: subchannel 0 quantised in LDS; in flight, in steady-state
    //      order: stage 1, B(0), stage 2
    Stage<KIND> st0, st1;
    v8i bA[NB], bB[NB];
    load_stage(st0, 0);
    quant_store(0, 0, st0);
    load_stage(st1, min(1, nkb - 1));
    __builtin_amdgcn_sched_barrier(0);
    load_b(bA, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(st0, min(2, nkb - 1));
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();

    int kb = 0;
    for (; kb + 1 < nkb; kb += 2) {
        step(kb, bA, bB, st1);
        step(kb + 1, bB, bA, st0);
    }
    if (kb < nkb) step(kb, bA, bB, st1);

    if constexpr (SWIGLU) {
        // ---- fused gate+up epilogue: h = silu(gate) * up, silu(z) = z / (1 + e^-z)
        //      (hardware exp and reciprocal: a few ulp, far inside the tolerance)
        float h[MB][2][4];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gt = acc[i][jj][r], up = acc[i][jj + 2][r];
                    h[i][jj][r] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                }
        if constexpr (OUT_BF16) {
            // through this wave's LDS block: 64-byte row segments, 4 lanes per row
            uint8_t (*ep)[SmemAll<WN>::kEpiRow] = smu.epi[wave];
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    *reinterpret_cast<uint2*>(&ep[16 * i + lr][(16 * jj + 4 * lc) * 2]) =
                        make_uint2(pack_bf16x2(h[i][jj][0], h[i][jj][1]), pack_bf16x2(h[i][jj][2], h[i][jj][3]));
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            const int orow = lane >> 2, ocol = (lane & 3) * 16;
#pragma unroll
            for (int q = 0; q < (TM + 15) / 16; ++q) {
                const int r = 16 * q + orow;
                const uint4 v = *reinterpret_cast<const uint4*>(&ep[r][ocol]);
                const int grow = row0 + r;
                if (grow >= it.lo && grow < it.hi)
                    store_out(reinterpret_cast<uint8_t*>(out) + ((int64_t)grow * N + ncol0) * 2 + ocol, v);
            }
        } else {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int grow = row0 + 16 * i + lr;
                if (grow < it.lo || grow >= it.hi) continue;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (int64_t)grow * N + ncol0 + 16 * jj + 4 * lc) =
                        make_float4(h[i][jj][0], h[i][jj][1], h[i][jj][2], h[i][jj][3]);
            }
        }
        if (q_out != nullptr) {
            // 1x128 quantisation of the fp32 activation for the next layer:
            // the block's row abs-max over the lane's 8 values, the row's 4
            // lanes and the 4 waves of the block (LDS), then the LHS recipe.
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                float m = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(h[i][jj][r]));
                m = fmaxf(m, __shfl_xor(m, 16, 64));
                m = fmaxf(m, __shfl_xor(m, 32, 64));
                if (lc == 0) s_rmax[wave][16 * i + lr] = m;
            }
            __syncthreads();
            const int w0 = (wave / 4) * 4;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const float a = fmaxf(fmaxf(s_rmax[w0][16 * i + lr], s_rmax[w0 + 1][16 * i + lr]),
                                      fmaxf(s_rmax[w0 + 2][16 * i + lr], s_rmax[w0 + 3][16 * i + lr]));
                const float sa = quant_scale(a);
                const float inv = quant_inv(sa);
                const int grow = row0 + 16 * i + lr;
                if (grow < it.lo || grow >= it.hi) continue;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    // 4-byte pieces of 16 rows per store: plain stores, which L2
                    // merges into whole lines (the non-temporal hint made each
                    // a partial-line write: 42.7 -> 44.3 us)
                    *reinterpret_cast<uint32_t*>(q_out + (int64_t)grow * N + ncol0 + 16 * jj + 4 * lc) =
                        e4m3x4(h[i][jj][0] * inv, h[i][jj][1] * inv, h[i][jj][2] * inv, h[i][jj][3] * inv);
                if (wave == w0 && lc == 0) s_out[(int64_t)grow * (N / kQBlock) + n0 / kQBlock + wave / 4] = sa;
            }
        }
        return;
    }

    // ---- epilogue.  bf16: each wave writes its 64 x WN block to its own LDS
    //      region (the loop's last barrier has retired every read of the A
    //      tiles) and stores it back row by row, 16 bytes per lane, so every
    //      store instruction writes whole WN*2-byte row segments.  fp32: each
    //      lane stores its 4 consecutive outputs directly.  Rows outside the
    //      item are skipped.
    if constexpr (OUT_BF16) {
        constexpr int ROWB = WN * 2;              // bytes of a row segment
        constexpr int LPRO = ROWB / 16;           // lanes per row on the way out
        constexpr int RPI = 64 / LPRO;            // rows per store instruction
        uint8_t (*ep)[SmemAll<WN>::kEpiRow] = smu.epi[wave];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                *reinterpret_cast<uint2*>(&ep[16 * i + lr][(16 * j + 4 * lc) * 2]) =
                    make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // this wave's writes before its reads
        const int orow = lane / LPRO, ocol = (lane % LPRO) * 16;
#pragma unroll
        for (int q = 0; q < (TM + RPI - 1) / RPI; ++q) {   // rows past the tile fail the row check
            const int r = RPI * q + orow;
            const uint4 v = *reinterpret_cast<const uint4*>(&ep[r][ocol]);
            const int grow = row0 + r;
            if (grow >= it.lo && grow < it.hi)
                store_out(reinterpret_cast<uint8_t*>(out) + ((int64_t)grow * N + ncol0) * 2 + ocol, v);
        }
    } else {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int grow = row0 + 16 * i + lr;
            if (grow < it.lo || grow >= it.hi) continue;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int64_t o = (int64_t)grow * N + ncol0 + 16 * j + 4 * lc;
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Warp-specialised variant for 512-column tiles.  Waves 0-3 (one per SIMD)
// are consumers: wave c owns output columns n0 + 128c .. +127 (one 128-column
// scale block), keeps its B operand in registers (reloading each 16-column
// block with the next subchannel right after its MFMAs) and only issues
// MFMAs and scale FMAs.  Waves 4-7 (one per SIMD) are producers: they load
// the raw LHS two subchannels ahead and quantise the next subchannel into
// the other LDS buffer.  Every SIMD thus has one wave feeding the matrix core
// and one feeding the VALU in the same step; one workgroup barrier per step,
// executed the same number of times by both roles (their loops are
// separate, so no role waits on the other's loads at a control-flow join).
// Producer lane (p, l): 16 values of each of rows 16p + l/8 and
// 16p + 8 + l/8 (runs at 8c and 64 + 8c, c = l % 8) — the same per-row
// recipe and lane layout as the plain kernel, two rows per lane.  NW = 16
// doubles both roles: 8 consumers of 64 columns (two per SIMD, one scale
// block per pair) and 8 producers of one row per lane (row 8p + l/8).
// Producers whose rows all lie past a 48-row tile only take the barriers.
//
// B4: MXFP4 weights ("实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1;
// OCP MX v1.0) in the packed order of quantize_rhs_mxfp4_kernel, TN = 512,
// 256 or 128 columns.  Each consumer block step loads 16 bytes of E2M1 codes
// and one E8M0 byte per lane and hands the byte to the MFMA as the first
// operand's scale, so the MFMA returns the MX-dequantised block product and
// the FMA factor is the LHS scale alone.  The producers store the LHS codes
// with K runs 1<->2 and 5<->6 of 16 exchanged (the MFMA's K grouping for an
// FP4 first operand, which the packed weights follow).
// I4: int4 weights (same sections: int4 is the other sub-byte RHS type) with
// the FP8 path's 128x128 fp32 block scales, packed at 16 bytes per lane and
// block step (quantize_rhs_int4_kernel), TN = 512, 256 or 128.  gfx950 has
// no MFMA taking int4, so each consumer expands its codes to E4M3 in
// registers (int4_to_e4m3x4: every int4 value is exact in E4M3) right before
// the block's MFMAs; the rest is the FP8 path.
template <int KIND, bool OUT_BF16, int TM, bool WRITE_Q, int NW = 8, int TN = 512, bool B4 = false,
          int NP = NW / 2, int BD = 1, bool I4 = false>
__global__ __launch_bounds__(64 * NW, NW / 4) void fp8_fwd_ws_kernel(   // TM = 48 (64 spills)
    const void* __restrict__ lhs, const float* __restrict__ lhs_scale,
    const uint8_t* __restrict__ rhs, const void* __restrict__ rhs_scale_v,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    uint8_t* __restrict__ q_out, float* __restrict__ s_out, int ntiles_n, int nblocks,
    int32_t* __restrict__ status, int placement) {
    static_assert(TM == 64 || TM == 48, "64- or 48-row tiles");
    static_assert(NW == 8 || NW == 12 || NW == 16, "8, 12 or 16 waves");
    static_assert(NP == 4 || NP == 8, "4 or 8 producer waves");
    static_assert((B4 || I4) ? (NW == 16 && NP == 8 && (TN == 512 || TN == 256 || TN == 128)) : TN == 512,
                  "FP8 weights: 512 columns; MXFP4 and int4: 16 waves, 512/256/128 columns");
    static_assert(!(B4 && I4), "one weight type");
    constexpr int MB = TM / 16;
    constexpr int NC = NW - NP;            // consumer waves
    static_assert(NC == 4 || NC == 8, "4 or 8 consumer waves");
    constexpr int CWID = TN / NC;          // output columns per consumer wave
    constexpr int NBC = CWID / 16;         // 16-column blocks per consumer wave
    constexpr int HP = 8 / NP;             // rows per producer lane
    const float* __restrict__ rhs_scale = reinterpret_cast<const float*>(rhs_scale_v);
    const uint8_t* __restrict__ rhs_e8 = reinterpret_cast<const uint8_t*>(rhs_scale_v);
    constexpr int kThr = 64 * NW;
    constexpr int OUT_BYTES = OUT_BF16 ? 2 : 4;
    constexpr int kEpiRow = CWID * OUT_BYTES + 16;  // staged output row (bytes)

    struct Tiles {
        uint8_t a[2][kTM][kLdsRow];
        float c[2][kLPR][kTM];
    };
    union SmemWs {
        Tiles t;
        uint8_t epi[NC][TM][kEpiRow];
    };
    __shared__ WorkItem s_item;
    __shared__ __attribute__((aligned(16))) SmemWs smw;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // placement 2: each group's items on one XCD (one column tile, G <= 64,
    // nblocks = 8 x slots); else consecutive items on one XCD
    // (the library picks this kernel when every item fits on the chip at
    // once, so the spare blocks of the consecutive mapping cost no time)
    const int L = placement == 2 ? 0 : xcd_remap(blockIdx.x, nblocks);
    const int nt = placement == 2 ? 0 : L % ntiles_n;
    if (wave == 0) {
        const WorkItem it = placement == 2
            ? group_aligned_work_item(group_sizes, G, M, TM, nblocks / kNumXcd, blockIdx.x)
            : find_work_item(group_sizes, G, M, TM, L / ntiles_n);
        if (lane == 0) s_item = it;
    } else if (wave == 1 && blockIdx.x == 0) {   // the call's device status word
        const int st = group_status(group_sizes, G, M);
        if (lane == 0) status[0] = st;
    }
    __syncthreads();
    const WorkItem it = s_item;
    if (it.g < 0) return;
    const int n0 = nt * TN;
    if (it.g == G) {  // rows past the last group: zeros
        const int rows = it.hi - it.lo;
        constexpr int V = 16 / OUT_BYTES;
        for (int e = tid; e < rows * (TN / V); e += kThr) {
            const int r = it.lo + e / (TN / V), c = n0 + (e % (TN / V)) * V;
            store_out(reinterpret_cast<uint8_t*>(out) + ((int64_t)r * N + c) * OUT_BYTES,
                make_uint4(0, 0, 0, 0));
        }
        return;
    }
    const int g = it.g, row0 = it.tile * TM;
    const int nkb = K / kTK, nnb = N / kQBlock;

    if (wave >= NC) {
        // ------------------------------------------------------ producer
        const int p = wave - NC;
        if (8 * HP * p >= TM) {
            // every row of this producer lies past the tile: only keep the
            // barrier count (prologue + one per step)
            for (int k = 0; k <= nkb; ++k) __syncthreads();
            return;
        }
        const int qchunk = lane % kLPR;
        int qrow[HP];
        int64_t qgrow[HP], qlrow[HP];
        bool qvalid[HP];
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            qrow[h] = 8 * HP * p + 8 * h + lane / kLPR;
            qgrow[h] = row0 + qrow[h];
            qvalid[h] = qgrow[h] >= it.lo && qgrow[h] < it.hi;
            qlrow[h] = qvalid[h] ? qgrow[h] : it.lo;
        }
        const float* srl = B4 ? nullptr : rhs_scale + (int64_t)g * nkb * nnb + n0 / kQBlock + min(qchunk, TN / kQBlock - 1);
        struct Stage2 {
            RawA<KIND> raw[HP];
            float sr;
        };
        auto load_stage = [&](Stage2& st, int kb) {
#pragma unroll
            for (int h = 0; h < HP; ++h) load_raw<KIND>(st.raw[h], lhs, lhs_scale, qlrow[h], K, kb, qchunk);
            if constexpr (!B4) st.sr = srl[kb * nnb];
        };
        // LDS position of the 8-byte run of codes k0 .. k0+7 of a row
        auto lds_pos = [](int k0) {
            if constexpr (!B4) return k0;
            const int r = (k0 >> 4) & 3;
            return (k0 & ~63) | ((r == 1 || r == 2 ? 3 - r : r) << 4) | (k0 & 15);
        };
        auto quant_store = [&](int kb, int buf, const Stage2& st) {
#pragma unroll
            for (int h = 0; h < HP; ++h) {
                uint2 codes[kNP];
                const float s = quantize_raw<KIND>(st.raw[h], codes);
#pragma unroll
                for (int q = 0; q < kNP; ++q)
                    *reinterpret_cast<uint2*>(&smw.t.a[buf][qrow[h]][lds_pos(qchunk * 8 + q * 8 * kLPR)]) = codes[q];
                if constexpr (B4) {
                    if (qchunk == 0) smw.t.c[buf][0][qrow[h]] = s;
                } else {
                    smw.t.c[buf][qchunk][qrow[h]] = s * st.sr;
                }
                if (WRITE_Q && nt == 0 && qvalid[h]) {
#pragma unroll
                    for (int q = 0; q < kNP; ++q)
                        *reinterpret_cast<uint2*>(q_out + qgrow[h] * K + kb * kTK + qchunk * 8 + q * 8 * kLPR) = codes[q];
                    if (qchunk == 0) s_out[qgrow[h] * nkb + kb] = s;
                }
            }
        };
        Stage2 st0, st1;
        load_stage(st0, 0);
        quant_store(0, 0, st0);
        load_stage(st1, min(1, nkb - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_stage(st0, min(2, nkb - 1));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // step k: quantise k+1 (loaded two steps ago) into buffer (k+1)&1,
        // reload that stage with k+3
        auto pstep = [&](int k, Stage2& sq) {
            quant_store(min(k + 1, nkb - 1), (k + 1) & 1, sq);
            load_stage(sq, min(k + 3, nkb - 1));
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        };
        int k = 0;
        for (; k + 1 < nkb; k += 2) {
            pstep(k, st1);
            pstep(k + 1, st0);
        }
        if (k < nkb) pstep(k, st1);
        return;
    }

    // ---------------------------------------------------------- consumer
    const int cw = wave;                          // 0 .. NC-1
    const int lr = lane & 15, lc = lane >> 4;
    const int ncol0 = n0 + CWID * cw;
    const int cslot = B4 ? 0 : (CWID * cw) / 128;   // the wave's 128-column scale block
    const uint8_t* bptr = rhs + ((int64_t)g * (N / 16) + ncol0 / 16) * nkb * (B4 || I4 ? 1024 : 2048) + lane * 16;
    const uint8_t* eptr = B4 ? rhs_e8 + ((int64_t)g * (N / 16) + ncol0 / 16) * nkb * 64 + lane : nullptr;
    v4f acc[MB][NBC];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBC; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // B of the next BD steps in registers: set s holds the steps k with
    // k % BD == s (the loop below runs steps in pairs, so s is static)
    v8i b[BD][NBC];
    int be[BD][NBC];
    auto load_b1 = [&](int s, int j, int kb) {
        if constexpr (B4 || I4) {
            const v4i lo = *reinterpret_cast<const v4i*>(bptr + ((int64_t)j * nkb + kb) * 1024);
            b[s][j] = __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
            if constexpr (B4) be[s][j] = eptr[((int64_t)j * nkb + kb) * 64];
        } else {
            const uint8_t* q = bptr + ((int64_t)j * nkb + kb) * 2048;
            const uint4 lo = *reinterpret_cast<const uint4*>(q);
            const uint4 hi = *reinterpret_cast<const uint4*>(q + 1024);
            b[s][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };
#pragma unroll
    for (int s = 0; s < BD; ++s)
#pragma unroll
        for (int j = 0; j < NBC; ++j) load_b1(s, j, min(s, nkb - 1));
    __syncthreads();
    // step k: fragments and factors of k from buffer k&1, MFMAs of k with B
    // set k % BD, each B block reloaded with step k+BD right after its MFMAs
    auto cstep = [&](int k, auto set) {
        constexpr int S = decltype(set)::value;
        v8i (&bs)[NBC] = b[S];
        int (&bes)[NBC] = be[S];
        const int buf = k & 1, k1 = min(k + BD, nkb - 1);
        v8i af[MB];
        float cf[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            af[i] = *reinterpret_cast<const v8i*>(&smw.t.a[buf][16 * i + lr][lc * 32]);
            cf[i] = smw.t.c[buf][cslot][16 * i + lr];
        }
#pragma unroll
        for (int j = 0; j < NBC; ++j) {
            v8i bj = bs[j];
            if constexpr (I4) {   // 32 int4 codes (4 dwords) -> 32 E4M3 codes (8 dwords)
#pragma unroll
                for (int d = 3; d >= 0; --d) {
                    const uint32_t x = (uint32_t)bs[j][d];
                    bj[2 * d] = (int)int4_to_e4m3x4(x);
                    bj[2 * d + 1] = (int)int4_to_e4m3x4(x >> 4);
                }
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                v4f pr;
                if constexpr (B4)   // first operand E2M1 with its E8M0 scale
                    pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bs[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, bes[j], 0, 127);
                else
                    pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bj, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], cf[i], acc[i][j][r]);
            }
            load_b1(S, j, k1);
        }
        __syncthreads();
    };
    int k = 0;
    for (; k + 1 < nkb; k += 2) {
        cstep(k, std::integral_constant<int, 0>{});
        cstep(k + 1, std::integral_constant<int, 1 % BD>{});
    }
    if (k < nkb) cstep(k, std::integral_constant<int, 0>{});

    // ---- epilogue: this wave's TM x CWID block through its LDS region (the
    //      last barrier retired every read of the A tiles), stored back as
    //      whole rows (256 bytes bf16 / 512 bytes fp32); rows outside the
    //      item are skipped
    uint8_t (*ep)[kEpiRow] = smw.epi[cw];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBC; ++j) {
            uint8_t* d = &ep[16 * i + lr][(16 * j + 4 * lc) * OUT_BYTES];
            if constexpr (OUT_BF16)
                *reinterpret_cast<uint2*>(d) =
                    make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
            else
                *reinterpret_cast<float4*>(d) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    constexpr int LPRO = CWID * OUT_BYTES / 16;  // lanes per row on the way out
    constexpr int RPI = 64 / LPRO;
    const int orow = lane / LPRO, ocol = (lane % LPRO) * 16;
#pragma unroll
    for (int q = 0; q < (TM + RPI - 1) / RPI; ++q) {
        const int r = RPI * q + orow;
        if (r >= TM) break;
        const uint4 v = *reinterpret_cast<const uint4*>(&ep[r][ocol]);
        const int grow = row0 + r;
        if (grow >= it.lo && grow < it.hi)
            store_out(reinterpret_cast<uint8_t*>(out) + ((int64_t)grow * N + ncol0) * OUT_BYTES + ocol, v);
    }
}

// ---------------------------------------------------------------------------
// Row-resident variant for wide, shallow shapes (N a multiple of 512 with
// several 512-column tiles, K <= 128 * KBM): one workgroup per 48-row item
// sweeps every 512-column tile of N.  The producers quantise the item's rows
// once, for all K, into LDS slots of their own (one per 128-K step), then
// exit; the consumers run the K loop once per column tile against those
// resident codes, streaming only the weights, and write each tile through
// their own LDS staging rows.  Compared with one workgroup per (item, tile)
// this quantises and loads the LHS once instead of N/512 times and pays one
// prologue per item.  16 waves (8 consumers of 64 columns, 8 producers of one
// row per lane).  The first column tile keeps one barrier per K step (step
// k's codes ready); its loop is separate from the later tiles', which have
// no barrier at all.  B4: MXFP4 weights as in fp8_fwd_ws_kernel (codes in
// the MFMA's FP4 K grouping, E8M0 scales on the MFMA, LHS scale on the FMA).
template <int KIND, bool OUT_BF16, int KBM, bool B4 = false, int TN = 512>
__global__ __launch_bounds__(1024, 4) void fp8_fwd_wsn_kernel(
    const void* __restrict__ lhs, const float* __restrict__ lhs_scale,
    const uint8_t* __restrict__ rhs, const void* __restrict__ rhs_scale_v,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    int nblocks, int32_t* __restrict__ status) {
    static_assert(TN == 512 || TN == 256, "512- or 256-column tiles");
    constexpr int TM = 48, MB = TM / 16, NC = 8, CWID = TN / NC, NBC = CWID / 16;
    constexpr int kThr = 1024;
    constexpr int OUT_BYTES = OUT_BF16 ? 2 : 4;
    constexpr int kEpiRow = CWID * OUT_BYTES + 16;
    const float* __restrict__ rhs_scale = reinterpret_cast<const float*>(rhs_scale_v);
    const uint8_t* __restrict__ rhs_e8 = reinterpret_cast<const uint8_t*>(rhs_scale_v);
    struct SmemRes {
        uint8_t a[KBM][TM][kLdsRow];     // resident codes, one slot per 128-K step
        float sa[KBM][TM];               // their 1x128 scales
        uint8_t epi[NC][TM][kEpiRow];    // per-consumer output staging
    };
    __shared__ WorkItem s_item;
    __shared__ __attribute__((aligned(16))) SmemRes sm;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (wave == 0) {
        // the items that exist, dealt evenly over the XCDs
        int col;
        const WorkItem it = balanced_work_item(group_sizes, G, M, TM, 1, blockIdx.x, col);
        if (lane == 0) s_item = it;
    } else if (wave == 1 && blockIdx.x == 0) {   // the call's device status word
        const int st = group_status(group_sizes, G, M);
        if (lane == 0) status[0] = st;
    }
    __syncthreads();
    const WorkItem it = s_item;
    if (it.g < 0) return;
    if (it.g == G) {  // rows past the last group: zeros over all N
        const int rows = it.hi - it.lo;
        const int per_row = N * OUT_BYTES / 16;
        for (int e = tid; e < rows * per_row; e += kThr) {
            const int r = it.lo + e / per_row, c = e % per_row;
            store_out(reinterpret_cast<uint8_t*>(out) + (int64_t)r * N * OUT_BYTES + c * 16,
                make_uint4(0, 0, 0, 0));
        }
        return;
    }
    const int g = it.g, row0 = it.tile * TM;
    const int nkb = K / kTK, nnb = N / kQBlock, ntiles = N / TN;

    if (wave >= NC) {
        // ------------------------------------------------------ producer
        const int p = wave - NC;
        if (8 * p >= TM) {
            for (int k = 0; k <= nkb; ++k) __syncthreads();
            return;
        }
        const int qchunk = lane % kLPR;
        const int qrow = 8 * p + lane / kLPR;
        const int64_t qgrow = row0 + qrow;
        const int64_t qlrow = qgrow >= it.lo && qgrow < it.hi ? qgrow : it.lo;
        // LDS position of the 8-byte run of codes k0 .. k0+7 of a row
        auto lds_pos = [](int k0) {
            if constexpr (!B4) return k0;
            const int r = (k0 >> 4) & 3;
            return (k0 & ~63) | ((r == 1 || r == 2 ? 3 - r : r) << 4) | (k0 & 15);
        };
        auto quant_store = [&](int kb, const RawA<KIND>& raw) {
            uint2 codes[kNP];
            const float s = quantize_raw<KIND>(raw, codes);
#pragma unroll
            for (int q = 0; q < kNP; ++q)
                *reinterpret_cast<uint2*>(&sm.a[kb][qrow][lds_pos(qchunk * 8 + q * 8 * kLPR)]) = codes[q];
            if (qchunk == 0) sm.sa[kb][qrow] = s;
        };
        RawA<KIND> st0, st1;
        load_raw<KIND>(st0, lhs, lhs_scale, qlrow, K, 0, qchunk);
        quant_store(0, st0);
        load_raw<KIND>(st1, lhs, lhs_scale, qlrow, K, min(1, nkb - 1), qchunk);
        __builtin_amdgcn_sched_barrier(0);
        load_raw<KIND>(st0, lhs, lhs_scale, qlrow, K, min(2, nkb - 1), qchunk);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // step k: quantise k+1 (loaded two steps ago) into its slot, reload
        // that stage with k+3
        auto pstep = [&](int k, RawA<KIND>& sq) {
            if (k + 1 < nkb) quant_store(k + 1, sq);
            load_raw<KIND>(sq, lhs, lhs_scale, qlrow, K, min(k + 3, nkb - 1), qchunk);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        };
        int k = 0;
        for (; k + 1 < nkb; k += 2) {
            pstep(k, st1);
            pstep(k + 1, st0);
        }
        if (k < nkb) pstep(k, st1);
        return;
    }

    // ---------------------------------------------------------- consumer
    const int cw = wave;
    const int lr = lane & 15, lc = lane >> 4;
    v4f acc[MB][NBC];
    v8i b[NBC];
    int be[NBC];
    // B block j of column tile t at K step kb: the expert's packed codes from
    // a scalar base, a wave-uniform 32-bit offset (one expert's codes are
    // N*K bytes, N*K/2 for MXFP4) and the lane's 16 bytes
    const uint8_t* __restrict__ rg = rhs + (int64_t)g * N * K / (B4 ? 2 : 1);
    const uint8_t* __restrict__ eg = B4 ? rhs_e8 + (int64_t)g * N * K / 32 : nullptr;
    const uint32_t lane_off = (uint32_t)lane * 16u;
    auto load_b1 = [&](int j, int t, int kb) {
        const uint32_t chunk = (uint32_t)__builtin_amdgcn_readfirstlane(
            ((t * TN + CWID * cw) / 16 + j) * nkb + kb);
        if constexpr (B4) {
            const v4i lo = *reinterpret_cast<const v4i*>(rg + (chunk * 1024u + lane_off));
            b[j] = __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
            be[j] = eg[chunk * 64u + (uint32_t)lane];
        } else {
            const uint4 lo = *reinterpret_cast<const uint4*>(rg + (chunk * 2048u + lane_off));
            const uint4 hi = *reinterpret_cast<const uint4*>(rg + (chunk * 2048u + 1024u + lane_off));
            b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };
#pragma unroll
    for (int j = 0; j < NBC; ++j) load_b1(j, 0, 0);
    __syncthreads();
    uint8_t (*ep)[kEpiRow] = sm.epi[cw];
    // one column tile: K loop (with the producers' step barrier on the first
    // tile only), then the epilogue through this wave's staging rows
    auto tile = [&](int t, auto first_tile) {
        constexpr bool FIRST = decltype(first_tile)::value;
        const int cslot = (t * TN + CWID * cw) / kQBlock;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NBC; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < nkb; ++kb) {
            const int nt = kb + 1 < nkb ? t : min(t + 1, ntiles - 1);
            const int nk = kb + 1 < nkb ? kb + 1 : (t + 1 < ntiles ? 0 : kb);
            const float sr = B4 ? 1.0f : rhs_scale[((int64_t)g * nkb + kb) * nnb + cslot];
            v8i af[MB];
            float cf[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                af[i] = *reinterpret_cast<const v8i*>(&sm.a[kb][16 * i + lr][lc * 32]);
                cf[i] = sm.sa[kb][16 * i + lr] * sr;
            }
#pragma unroll
            for (int j = 0; j < NBC; ++j) {
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    v4f pr;
                    if constexpr (B4)
                        pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            b[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, be[j], 0, 127);
                    else
                        pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            b[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], cf[i], acc[i][j][r]);
                }
                load_b1(j, nt, nk);
            }
            if constexpr (FIRST) __syncthreads();   // step kb + 1's codes ready
        }
        const int ncol0 = t * TN + CWID * cw;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NBC; ++j) {
                uint8_t* d = &ep[16 * i + lr][(16 * j + 4 * lc) * OUT_BYTES];
                if constexpr (OUT_BF16)
                    *reinterpret_cast<uint2*>(d) =
                        make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
                else
                    *reinterpret_cast<float4*>(d) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        constexpr int LPRO = CWID * OUT_BYTES / 16;
        constexpr int RPI = 64 / LPRO;
        const int orow = lane / LPRO, ocol = (lane % LPRO) * 16;
        // FP8 weights: the destination is a wave-uniform base per store plus
        // one per-lane byte offset, so no per-row 64-bit address stays live
        // across the tile loop (spilled, its reload made every store wait for
        // all outstanding memory operations, the next tile's weights
        // included).  MXFP4 keeps per-row addresses: the other form moves
        // its register pressure into the K loop.
        const uint32_t olane = (uint32_t)orow * (uint32_t)N * OUT_BYTES + (uint32_t)ocol;
        uint8_t* const obase = reinterpret_cast<uint8_t*>(out) + ((int64_t)row0 * N + ncol0) * OUT_BYTES;
#pragma unroll
        for (int q = 0; q < (TM + RPI - 1) / RPI; ++q) {
            const int r = RPI * q + orow;
            if (r >= TM) break;
            const uint4 v = *reinterpret_cast<const uint4*>(&ep[r][ocol]);
            const int grow = row0 + r;
            if (grow >= it.lo && grow < it.hi) {
                if constexpr (B4 && !FIRST && OUT_BF16)
                    store_out(reinterpret_cast<uint8_t*>(out) + ((int64_t)grow * N + ncol0) * OUT_BYTES + ocol, v);
                else
                    store_out(obase + (int64_t)(RPI * q) * N * OUT_BYTES + olane, v);
            }
        }
        // the staging rows are rewritten by the next tile's epilogue only
        // after this wave's reads above (program order within the wave)
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };
    tile(0, std::true_type{});
    for (int t = 1; t < ntiles; ++t) tile(t, std::false_type{});
}

// The row-resident kernel addresses one expert's weights with 32-bit byte
// offsets (at most N*K bytes of codes), so it runs only when they fit.
inline bool wsn_offsets_fit(int K, int N) { return (int64_t)N * K < (int64_t(1) << 32); }

template <int KIND, int KBM, bool B4 = false, int TN = 512>
hipError_t launch_wsn(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                      const void* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                      int G, void* out, bool out_bf16, int32_t* status, hipStream_t stream) {
    const int nblocks = (int)max_work_items(M, G, 48);
    // LDS of the fp32-output form: resident codes and scales plus fp32
    // staging rows; beyond the 160 KB of a CU only bf16 output is offered
    constexpr int kF32Lds = KBM * 48 * (kLdsRow + 4) + 8 * 48 * ((TN / 8) * 4 + 16);
    if constexpr (kF32Lds > 160 * 1024) {
        if (!out_bf16) return hipErrorInvalidValue;
        hipLaunchKernelGGL((fp8_fwd_wsn_kernel<KIND, true, KBM, B4, TN>), dim3(nblocks), dim3(1024), 0,
                           stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                           nblocks, status);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((fp8_fwd_wsn_kernel<KIND, true, KBM, B4, TN>), dim3(nblocks), dim3(1024),
                               0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                               nblocks, status);
        else
            hipLaunchKernelGGL((fp8_fwd_wsn_kernel<KIND, false, KBM, B4, TN>), dim3(nblocks), dim3(1024),
                               0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                               nblocks, status);
    }
    return hipGetLastError();
}

template <int KIND, int TM, bool WRITE_Q, int NW = 8, int TN = 512, bool B4 = false, int NP = NW / 2,
          int BD = 1, bool I4 = false>
hipError_t launch_ws(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                     const void* rhs_scale, const int32_t* group_sizes, int M, int K, int N, int G,
                     void* out, bool out_bf16, uint8_t* q_out, float* scale_out, int32_t* status, hipStream_t stream,
                     int placement = 1) {
    const int ntiles_n = N / TN;
    const int64_t items = max_work_items(M, G, TM);
    // group-aligned placement: kNumXcd x slots blocks, slots >= ceil(items / 8)
    const int nblocks = placement == 2
        ? kNumXcd * (int)std::max<int64_t>((items + kNumXcd - 1) / kNumXcd, device_cus() / kNumXcd)
        : (int)(items * ntiles_n);
    if (out_bf16)
        hipLaunchKernelGGL((fp8_fwd_ws_kernel<KIND, true, TM, WRITE_Q, NW, TN, B4, NP, BD, I4>), dim3(nblocks),
                           dim3(64 * NW), 0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M,
                           K, N, G, out, q_out, scale_out, ntiles_n, nblocks, status, placement);
    else
        hipLaunchKernelGGL((fp8_fwd_ws_kernel<KIND, false, TM, WRITE_Q, NW, TN, B4, NP, BD, I4>), dim3(nblocks),
                           dim3(64 * NW), 0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M,
                           K, N, G, out, q_out, scale_out, ntiles_n, nblocks, status, placement);
    return hipGetLastError();
}

// MXFP4 weights: the row-resident sweep (wide, shallow shapes) or the
// warp-specialised kernel with 48-row tiles of cfg.tile_n columns.
template <int KIND>
hipError_t launch_mxfp4_kind(const TileConfig& cfg, const void* lhs, const float* lhs_scale,
                             const uint8_t* rhs_q, const uint8_t* rhs_e8, const int32_t* group_sizes,
                             int M, int K, int N, int G, void* out, bool out_bf16, int32_t* status,
                             hipStream_t stream) {
    if (cfg.kernel == kKerRowResident) {
        if (K <= 512)
            return launch_wsn<KIND, 4, true>(lhs, lhs_scale, rhs_q, rhs_e8, group_sizes, M, K, N, G,
                                             out, out_bf16, status, stream);
        return launch_wsn<KIND, 8, true>(lhs, lhs_scale, rhs_q, rhs_e8, group_sizes, M, K, N, G, out,
                                         out_bf16, status, stream);
    }
    if (cfg.tile_n == 512)
        return launch_ws<KIND, 48, false, 16, 512, true>(lhs, lhs_scale, rhs_q, rhs_e8, group_sizes,
                                                         M, K, N, G, out, out_bf16, nullptr,
                                                         nullptr, status, stream);
    if (cfg.tile_n == 256)
        return launch_ws<KIND, 48, false, 16, 256, true>(lhs, lhs_scale, rhs_q, rhs_e8, group_sizes,
                                                         M, K, N, G, out, out_bf16, nullptr,
                                                         nullptr, status, stream);
    return launch_ws<KIND, 48, false, 16, 128, true>(lhs, lhs_scale, rhs_q, rhs_e8, group_sizes, M,
                                                     K, N, G, out, out_bf16, nullptr, nullptr,
                                                     status, stream);
}

// int4 weights: the warp-specialised kernel with 48-row tiles of cfg.tile_n
// columns.
template <int KIND>
hipError_t launch_int4_kind(const TileConfig& cfg, const void* lhs, const float* lhs_scale,
                            const uint8_t* rhs_q, const float* rhs_scale, const int32_t* group_sizes,
                            int M, int K, int N, int G, void* out, bool out_bf16, int32_t* status,
                            hipStream_t stream) {
    if (cfg.tile_n == 512)
        return launch_ws<KIND, 48, false, 16, 512, false, 8, 1, true>(lhs, lhs_scale, rhs_q, rhs_scale,
                                                                      group_sizes, M, K, N, G, out, out_bf16,
                                                                      nullptr, nullptr, status, stream);
    if (cfg.tile_n == 256)
        return launch_ws<KIND, 48, false, 16, 256, false, 8, 1, true>(lhs, lhs_scale, rhs_q, rhs_scale,
                                                                      group_sizes, M, K, N, G, out, out_bf16,
                                                                      nullptr, nullptr, status, stream);
    return launch_ws<KIND, 48, false, 16, 128, false, 8, 1, true>(lhs, lhs_scale, rhs_q, rhs_scale,
                                                                  group_sizes, M, K, N, G, out, out_bf16,
                                                                  nullptr, nullptr, status, stream);
}

template <int KIND, int WN, int TM, bool WRITE_Q, bool SWIGLU = false>
hipError_t launch_cfg(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                      const float* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                      int G, void* out, bool out_bf16, uint8_t* q_out, float* scale_out,
                      int32_t* status, hipStream_t stream) {
    const int ntiles_n = N / (SWIGLU ? kWaves * WN / 2 : kWaves * WN);
    const int64_t items = max_work_items(M, G, TM);
    const int nblocks = (int)(items * ntiles_n);
    if (out_bf16)
        hipLaunchKernelGGL((fp8_fwd_kernel<KIND, true, WN, TM, WRITE_Q, SWIGLU>), dim3(nblocks), dim3(kThreads),
                           0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                           q_out, scale_out, ntiles_n, nblocks, status);
    else
        hipLaunchKernelGGL((fp8_fwd_kernel<KIND, false, WN, TM, WRITE_Q, SWIGLU>), dim3(nblocks), dim3(kThreads),
                           0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                           q_out, scale_out, ntiles_n, nblocks, status);
    return hipGetLastError();
}

template <int KIND, int WN, int TM>
hipError_t launch_wn(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                     const float* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                     int G, void* out, bool out_bf16, uint8_t* q_out, float* scale_out,
                     int32_t* status, hipStream_t stream) {
    if constexpr (KIND != kLhsE4M3) {
        if (q_out != nullptr)
            return launch_cfg<KIND, WN, TM, true>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K,
                                                  N, G, out, out_bf16, q_out, scale_out, status, stream);
    }
    return launch_cfg<KIND, WN, TM, false>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N,
                                           G, out, out_bf16, q_out, scale_out, status, stream);
}

// The FP8 forward with a resolved configuration (gmm_config.cpp: the
// row-resident sweep for wide, shallow shapes; 48 x 512 tiles on the
// warp-specialised kernel when even the worst-case grid fits the chip at
// once; else the uniform kernel with the widest column tile dividing N).
template <int KIND>
hipError_t launch_kind(const TileConfig& cfg, const void* lhs, const float* lhs_scale,
                       const uint8_t* rhs, const float* rhs_scale, const int32_t* group_sizes,
                       int M, int K, int N, int G, void* out, bool out_bf16, uint8_t* q_out,
                       float* scale_out, int32_t* status, hipStream_t stream) {
    const bool write_q = KIND != kLhsE4M3 && q_out != nullptr;
    if (cfg.kernel == kKerRowResident) {
        if (cfg.tile_n == 256)
            return launch_wsn<KIND, 16, false, 256>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K,
                                                    N, G, out, out_bf16, status, stream);
        if (K <= 512)
            return launch_wsn<KIND, 4>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                                       out_bf16, status, stream);
        return launch_wsn<KIND, 8>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                                   out_bf16, status, stream);
    }
    if (cfg.kernel == kKerWs) {
        if (write_q)
            return launch_ws<KIND, 48, true>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G,
                                             out, out_bf16, q_out, scale_out, status, stream);
        if (cfg.waves == 16)
            return launch_ws<KIND, 48, false, 16>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N,
                                                  G, out, out_bf16, nullptr, nullptr, status, stream,
                                                  cfg.placement);
        if (cfg.waves == 12 && cfg.depth == 2)
            return launch_ws<KIND, 48, false, 12, 512, false, 4, 2>(
                lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out, out_bf16, nullptr,
                nullptr, status, stream);
        if (cfg.waves == 12)
            return launch_ws<KIND, 48, false, 12, 512, false, 4>(lhs, lhs_scale, rhs, rhs_scale,
                                                                 group_sizes, M, K, N, G, out,
                                                                 out_bf16, nullptr, nullptr, status,
                                                                 stream);
        return launch_ws<KIND, 48, false>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G,
                                          out, out_bf16, nullptr, nullptr, status, stream);
    }
    const int wn = cfg.tile_n / kWaves;
#define GMM_FP8_WN_TM(WN_, TM_)                                                                  \
    if (wn == WN_ && cfg.tile_m == TM_)                                                          \
        return launch_wn<KIND, WN_, TM_>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, \
                                         out, out_bf16, q_out, scale_out, status, stream);
    GMM_FP8_WN_TM(64, 64)
    GMM_FP8_WN_TM(64, 48)
    GMM_FP8_WN_TM(32, 64)
    GMM_FP8_WN_TM(32, 48)
    GMM_FP8_WN_TM(16, 48)
#undef GMM_FP8_WN_TM
    return launch_wn<KIND, 16, 64>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                                   out_bf16, q_out, scale_out, status, stream);
}

// Fused gate+up: 256 output columns per workgroup, cfg.tile_m rows.
template <int KIND>
hipError_t launch_swiglu_kind(const TileConfig& cfg, const void* lhs, const float* lhs_scale,
                              const uint8_t* rhs, const float* rhs_scale, const int32_t* group_sizes,
                              int M, int K, int N, int G, void* out, bool out_bf16, uint8_t* act_q,
                              float* act_scale, int32_t* status, hipStream_t stream) {
    if (cfg.tile_m == 48)
        return launch_cfg<KIND, 64, 48, false, true>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M,
                                                     K, N, G, out, out_bf16, act_q, act_scale, status, stream);
    return launch_cfg<KIND, 64, 64, false, true>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K,
                                                 N, G, out, out_bf16, act_q, act_scale, status, stream);
}

}  // namespace

hipError_t launch_fp8_fwd_swiglu(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                                 const uint8_t* rhs, const float* rhs_scale,
                                 const int32_t* group_sizes, int M, int K, int N, int G,
                                 void* out, bool out_bf16, uint8_t* act_q, float* act_scale,
                                 int32_t* status, hipStream_t stream) {
    switch (lhs_kind) {
        case kLhsE4M3:
            return launch_swiglu_kind<kLhsE4M3>(cfg, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N,
                                                G, out, out_bf16, act_q, act_scale, status, stream);
        case kLhsBF16:
            return launch_swiglu_kind<kLhsBF16>(cfg, lhs, nullptr, rhs, rhs_scale, group_sizes, M, K, N,
                                                G, out, out_bf16, act_q, act_scale, status, stream);
        default:
            return launch_swiglu_kind<kLhsF32>(cfg, lhs, nullptr, rhs, rhs_scale, group_sizes, M, K, N,
                                               G, out, out_bf16, act_q, act_scale, status, stream);
    }
}

hipError_t launch_fp8_mxfp4_fwd(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                                const uint8_t* rhs_q, const uint8_t* rhs_scale,
                                const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                                bool out_bf16, int32_t* status, hipStream_t stream) {
    switch (lhs_kind) {
        case kLhsE4M3:
            return launch_mxfp4_kind<kLhsE4M3>(cfg, lhs, lhs_scale, rhs_q, rhs_scale, group_sizes, M, K,
                                               N, G, out, out_bf16, status, stream);
        case kLhsBF16:
            return launch_mxfp4_kind<kLhsBF16>(cfg, lhs, nullptr, rhs_q, rhs_scale, group_sizes, M, K, N,
                                               G, out, out_bf16, status, stream);
        default:
            return launch_mxfp4_kind<kLhsF32>(cfg, lhs, nullptr, rhs_q, rhs_scale, group_sizes, M, K, N,
                                              G, out, out_bf16, status, stream);
    }
}

hipError_t launch_fp8_int4_fwd(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                               const uint8_t* rhs_q, const float* rhs_scale,
                               const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                               bool out_bf16, int32_t* status, hipStream_t stream) {
    switch (lhs_kind) {
        case kLhsE4M3:
            return launch_int4_kind<kLhsE4M3>(cfg, lhs, lhs_scale, rhs_q, rhs_scale, group_sizes, M, K, N, G,
                                              out, out_bf16, status, stream);
        case kLhsBF16:
            return launch_int4_kind<kLhsBF16>(cfg, lhs, nullptr, rhs_q, rhs_scale, group_sizes, M, K, N, G,
                                              out, out_bf16, status, stream);
        default:
            return launch_int4_kind<kLhsF32>(cfg, lhs, nullptr, rhs_q, rhs_scale, group_sizes, M, K, N, G,
                                             out, out_bf16, status, stream);
    }
}

hipError_t launch_fp8_fwd(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                          const uint8_t* rhs, const float* rhs_scale,
                          const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                          bool out_bf16, uint8_t* q_out, float* scale_out, int32_t* status, hipStream_t stream) {
    switch (lhs_kind) {
        case kLhsE4M3:
            return launch_kind<kLhsE4M3>(cfg, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G,
                                         out, out_bf16, nullptr, nullptr, status, stream);
        case kLhsBF16:
            return launch_kind<kLhsBF16>(cfg, lhs, nullptr, rhs, rhs_scale, group_sizes, M, K, N, G,
                                         out, out_bf16, q_out, scale_out, status, stream);
        default:
            return launch_kind<kLhsF32>(cfg, lhs, nullptr, rhs, rhs_scale, group_sizes, M, K, N, G,
                                        out, out_bf16, q_out, scale_out, status, stream);
    }
}

}  // namespace gmm
