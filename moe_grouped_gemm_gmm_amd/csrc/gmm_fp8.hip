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
//    two waves share B, so it never goes through LDS.  Each column block is
//    reloaded with the next subchannel as soon as its MFMAs are issued.
//  - Raw A is loaded two subchannels ahead and quantised one ahead of the
//    MFMAs that use it; one barrier per subchannel.  The loop body has no
//    branches (prefetch indices are clamped), so loads stay in flight across
//    iterations instead of being drained at control-flow joins.
//  - Each 16x16 block is one v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0
//    scales: the FP8 products are exact) into a zero temporary, folded into
//    the fp32 accumulator with one FMA per element: acc += p * (sl * sr).
//  - The MFMA operands are swapped so every 16x16 block comes out transposed:
//    a lane owns one output row and four consecutive columns, which makes the
//    row factor one scalar per block and lets the epilogue store 8-byte (bf16)
//    or 16-byte (fp32) runs directly.
#include "gmm_device.hpp"
#include "gmm_launch.hpp"

#include <cstdio>
#include <cstdlib>

namespace gmm {

namespace {

constexpr int kTM = 64;            // rows per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTK = 128;           // one subchannel
constexpr int kLdsRow = kTK + 16;  // 144-byte LDS rows: conflict-free 16-lane ds_read_b128

enum LhsKind { kLhsE4M3 = 0, kLhsBF16 = 1, kLhsF32 = 2 };

// Raw LHS registers of one subchannel for this lane: one row, K values
// 8c..8c+7 and 64+8c..64+8c+7 (c = lane % 8), so that each load instruction of
// the wave reads the same 128-byte half of 8 rows.  Lanes of rows outside the
// work item load a clamped in-bounds row; their codes only reach output rows
// that are never stored.
template <int KIND>
struct RawA;
template <>
struct RawA<kLhsBF16> { uint4 d[2]; };
template <>
struct RawA<kLhsF32> { uint4 d[4]; };
template <>
struct RawA<kLhsE4M3> { uint2 d[2]; float s; };

template <int KIND>
__device__ __forceinline__ void load_raw(RawA<KIND>& r, const void* __restrict__ lhs,
                                         const float* __restrict__ lhs_scale, int64_t row, int K,
                                         int kb, int chunk) {
    const int64_t e = row * K + kb * kTK + chunk * 8;
    if constexpr (KIND == kLhsBF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(lhs) + e;
        r.d[0] = *reinterpret_cast<const uint4*>(p);
        r.d[1] = *reinterpret_cast<const uint4*>(p + 64);
    } else if constexpr (KIND == kLhsF32) {
        const float* p = reinterpret_cast<const float*>(lhs) + e;
        r.d[0] = *reinterpret_cast<const uint4*>(p);
        r.d[1] = *reinterpret_cast<const uint4*>(p + 4);
        r.d[2] = *reinterpret_cast<const uint4*>(p + 64);
        r.d[3] = *reinterpret_cast<const uint4*>(p + 68);
    } else {
        const uint8_t* p = reinterpret_cast<const uint8_t*>(lhs) + e;
        r.d[0] = *reinterpret_cast<const uint2*>(p);
        r.d[1] = *reinterpret_cast<const uint2*>(p + 64);
        r.s = lhs_scale[row * (K / kTK) + kb];
    }
}

// 16 values -> 16 codes (two 8-byte runs) and the row's scale; the abs-max is
// reduced over the 8 lanes that hold the row (DPP, no LDS round trip).
template <int KIND>
__device__ __forceinline__ float quantize_raw(const RawA<KIND>& r, uint2 (&codes)[2]) {
    if constexpr (KIND == kLhsE4M3) {
        codes[0] = r.d[0];
        codes[1] = r.d[1];
        return r.s;
    } else {
        float v[16];
        if constexpr (KIND == kLhsBF16) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                v[8 * q + 0] = bf16_lo(r.d[q].x); v[8 * q + 1] = bf16_hi(r.d[q].x);
                v[8 * q + 2] = bf16_lo(r.d[q].y); v[8 * q + 3] = bf16_hi(r.d[q].y);
                v[8 * q + 4] = bf16_lo(r.d[q].z); v[8 * q + 5] = bf16_hi(r.d[q].z);
                v[8 * q + 6] = bf16_lo(r.d[q].w); v[8 * q + 7] = bf16_hi(r.d[q].w);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[4 * q + 0] = __uint_as_float(r.d[q].x); v[4 * q + 1] = __uint_as_float(r.d[q].y);
                v[4 * q + 2] = __uint_as_float(r.d[q].z); v[4 * q + 3] = __uint_as_float(r.d[q].w);
            }
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
        a = max_over_8(a);
        const float s = quant_scale(a);
        const float inv = quant_inv(s);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
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
    uint8_t a[2][kTM][kLdsRow];         // E4M3 codes of the current and next subchannel
    float c[2][NBLK][kTM];              // sl[row] * sr[n-block]
};

template <int KIND, bool OUT_BF16, int WN, bool WRITE_Q>
__global__ __launch_bounds__(kThreads, WN <= 32 ? 2 : 1) void fp8_fwd_kernel(
    const void* __restrict__ lhs, const float* __restrict__ lhs_scale,
    const uint8_t* __restrict__ rhs, const float* __restrict__ rhs_scale,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    uint8_t* __restrict__ q_out, float* __restrict__ s_out, int ntiles_n, int nblocks) {
    constexpr int MB = kTM / 16;  // 16-row blocks
    constexpr int NB = WN / 16;   // 16-column blocks per wave
    constexpr int TN = kWaves * WN;
    constexpr int NBLK = Smem<WN>::NBLK;
    constexpr int OUT_BYTES = OUT_BF16 ? 2 : 4;

    __shared__ WorkItem s_item;
    __shared__ __attribute__((aligned(16))) Smem<WN> sm;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = xcd_remap(blockIdx.x, nblocks);
    const int w = L / ntiles_n, nt = L % ntiles_n;
    if (wave == 0) {
        const WorkItem it = find_work_item(group_sizes, G, M, 6, w);
        if (lane == 0) s_item = it;
    }
    __syncthreads();
    const WorkItem it = s_item;
    if (it.g < 0) return;
    const int n0 = nt * TN;

    if (it.g == G) {  // rows past the last group: zeros
        const int rows = it.hi - it.lo;
        constexpr int V = 16 / OUT_BYTES;  // elements per 16-byte store
        for (int e = tid; e < rows * (TN / V); e += kThreads) {
            const int r = it.lo + e / (TN / V), c = n0 + (e % (TN / V)) * V;
            *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(out) + ((int64_t)r * N + c) * OUT_BYTES) =
                make_uint4(0, 0, 0, 0);
        }
        return;
    }

    const int g = it.g, row0 = it.tile * kTM;
    const int nkb = K / kTK, nnb = N / kQBlock;

    // ---- quantiser role: row 8*wave + lane/8, K values 8c..8c+7 and
    //      64+8c..64+8c+7 with c = lane % 8
    const int qchunk = lane & 7;
    const int qrow = 8 * wave + (lane >> 3);
    const int64_t qgrow = row0 + qrow;
    const bool qvalid = qgrow >= it.lo && qgrow < it.hi;
    const int64_t qlrow = qvalid ? qgrow : it.lo;    // in-bounds row the loads use
    const bool write_q = WRITE_Q && nt == 0 && qvalid;
    const float* srg = rhs_scale + (int64_t)g * nkb * nnb + n0 / kQBlock;  // + kb*nnb + nblk

    // ---- MFMA role: columns [n0 + wave*WN, +WN); lane = row/col lr, K chunk lc.
    //      B is the packed RHS: 2 KB per (16-column block, subchannel), this
    //      lane's 32 codes at byte lane*16 of each 1 KB half.
    const int lr = lane & 15, lc = lane >> 4;
    const int ncol0 = n0 + wave * WN;
    const int my_nblk = (wave * WN) / 128;
    const uint8_t* bptr = rhs + ((int64_t)g * (N / 16) + ncol0 / 16) * nkb * 2048 + lane * 16;

    v4f acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    RawA<KIND> raw;
    v8i b[NB];

    // Quantise the raw registers (subchannel kb) into LDS buffer buf.  The
    // RHS scales of the tile's 128-column blocks are wave-uniform scalar loads.
    auto quant_store = [&](int kb, int buf) {
        const float* srk = srg + kb * nnb;   // wave-uniform: scalar loads
        float srv[NBLK];
#pragma unroll
        for (int q = 0; q < NBLK; ++q) srv[q] = srk[q];
        float sr = srv[0];
#pragma unroll
        for (int q = 1; q < NBLK; ++q) sr = qchunk == q ? srv[q] : sr;
        uint2 codes[2];
        const float s = quantize_raw<KIND>(raw, codes);
        *reinterpret_cast<uint2*>(&sm.a[buf][qrow][qchunk * 8]) = codes[0];
        *reinterpret_cast<uint2*>(&sm.a[buf][qrow][64 + qchunk * 8]) = codes[1];
        if (qchunk < NBLK) sm.c[buf][qchunk][qrow] = s * sr;
        if (write_q) {
            *reinterpret_cast<uint2*>(q_out + qgrow * K + kb * kTK + qchunk * 8) = codes[0];
            *reinterpret_cast<uint2*>(q_out + qgrow * K + kb * kTK + 64 + qchunk * 8) = codes[1];
            if (qchunk == 0) s_out[qgrow * nkb + kb] = s;
        }
    };
    auto load_b = [&](int j, int kb) {
        const uint8_t* p = bptr + ((int64_t)j * nkb + kb) * 2048;
        const uint4 lo = *reinterpret_cast<const uint4*>(p);
        const uint4 hi = *reinterpret_cast<const uint4*>(p + 1024);
        b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    // ---- prologue: subchannel 0 quantised in LDS, raw subchannel 1 and B(0) in registers
    load_raw<KIND>(raw, lhs, lhs_scale, qlrow, K, 0, qchunk);
#pragma unroll
    for (int j = 0; j < NB; ++j) load_b(j, 0);
    quant_store(0, 0);
    load_raw<KIND>(raw, lhs, lhs_scale, qlrow, K, min(1, nkb - 1), qchunk);
    __syncthreads();

    // Iteration kb (straight-line code, so loads stay in flight across it):
    // MFMAs of kb from LDS buffer kb&1, each B column block reloaded with
    // kb+1 right after its MFMAs; raw(kb+1) quantised into buffer (kb+1)&1;
    // raw(kb+2) loads issued.  Prefetch indices are clamped to the last
    // subchannel (a redundant reload) instead of branching.
    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        const int kb1 = min(kb + 1, nkb - 1), kb2 = min(kb + 2, nkb - 1);
        // Operands are swapped so each 16x16 block comes out transposed: lane
        // (lr, lc) holds row 16i + lr and the four consecutive columns
        // 16j + 4lc .. +3, so its per-row factor sl * sr is one scalar per row
        // block.
        v8i af[MB];
        float cf[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            af[i] = *reinterpret_cast<const v8i*>(&sm.a[buf][16 * i + lr][lc * 32]);
            cf[i] = sm.c[buf][my_nblk][16 * i + lr];
        }
        quant_store(kb1, buf ^ 1);
        load_raw<KIND>(raw, lhs, lhs_scale, qlrow, K, kb2, qchunk);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    b[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], cf[i], acc[i][j][r]);
            }
            load_b(j, kb1);
        }
        __syncthreads();
    }

    // ---- epilogue: each lane stores 4 consecutive outputs of its rows directly
    //      (8 bytes for bf16, 16 for fp32); rows outside the item are skipped
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int grow = row0 + 16 * i + lr;
        if (grow < it.lo || grow >= it.hi) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t o = (int64_t)grow * N + ncol0 + 16 * j + 4 * lc;
            if constexpr (OUT_BF16)
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + o) =
                    make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
            else
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

template <int KIND, int WN, bool WRITE_Q>
hipError_t launch_cfg(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                      const float* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                      int G, void* out, bool out_bf16, uint8_t* q_out, float* scale_out,
                      hipStream_t stream) {
    const int ntiles_n = N / (kWaves * WN);
    const int64_t items = max_work_items(M, G, kTM);
    const int nblocks = (int)(items * ntiles_n);
    if (out_bf16)
        hipLaunchKernelGGL((fp8_fwd_kernel<KIND, true, WN, WRITE_Q>), dim3(nblocks), dim3(kThreads),
                           0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                           q_out, scale_out, ntiles_n, nblocks);
    else
        hipLaunchKernelGGL((fp8_fwd_kernel<KIND, false, WN, WRITE_Q>), dim3(nblocks), dim3(kThreads),
                           0, stream, lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                           q_out, scale_out, ntiles_n, nblocks);
    return hipGetLastError();
}

template <int KIND, int WN>
hipError_t launch_wn(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                     const float* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                     int G, void* out, bool out_bf16, uint8_t* q_out, float* scale_out,
                     hipStream_t stream) {
    if (KIND != kLhsE4M3 && q_out != nullptr)
        return launch_cfg<KIND, WN, true>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G,
                                          out, out_bf16, q_out, scale_out, stream);
    return launch_cfg<KIND, WN, false>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G,
                                       out, out_bf16, q_out, scale_out, stream);
}

// Tile width: the widest of 512/256/128 columns that divides N (fewest
// re-quantisations of each LHS row).  GMM_FP8_WN=<16|32|64> overrides the
// per-wave width (tuning sweeps only).
template <int KIND>
hipError_t launch_kind(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                       const float* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                       int G, void* out, bool out_bf16, uint8_t* q_out, float* scale_out,
                       hipStream_t stream) {
    static const int forced = [] {
        const char* e = std::getenv("GMM_FP8_WN");
        return e ? std::atoi(e) : 0;
    }();
    int wn = N % 512 == 0 ? 64 : (N % 256 == 0 ? 32 : 16);
    if ((forced == 16 || forced == 32 || forced == 64) && N % (kWaves * forced) == 0) wn = forced;
    if (wn == 64)
        return launch_wn<KIND, 64>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                                    out_bf16, q_out, scale_out, stream);
    if (wn == 32)
        return launch_wn<KIND, 32>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                                    out_bf16, q_out, scale_out, stream);
    return launch_wn<KIND, 16>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                                out_bf16, q_out, scale_out, stream);
}

}  // namespace

hipError_t launch_fp8_fwd(const void* lhs, int lhs_kind, const float* lhs_scale,
                          const uint8_t* rhs, const float* rhs_scale,
                          const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                          bool out_bf16, uint8_t* q_out, float* scale_out, hipStream_t stream) {
    switch (lhs_kind) {
        case kLhsE4M3:
            return launch_kind<kLhsE4M3>(lhs, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G,
                                         out, out_bf16, nullptr, nullptr, stream);
        case kLhsBF16:
            return launch_kind<kLhsBF16>(lhs, nullptr, rhs, rhs_scale, group_sizes, M, K, N, G,
                                         out, out_bf16, q_out, scale_out, stream);
        default:
            return launch_kind<kLhsF32>(lhs, nullptr, rhs, rhs_scale, group_sizes, M, K, N, G,
                                        out, out_bf16, q_out, scale_out, stream);
    }
}

}  // namespace gmm
