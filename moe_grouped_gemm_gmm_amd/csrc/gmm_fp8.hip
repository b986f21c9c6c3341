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
// their scales.  The RHS is E4M3 codes stored K-contiguous per expert
// ([G,N,K]) with 128x128 block scales.
//
// One workgroup (4 waves) computes a 128x128 output tile of one work item
// (an expert's rows within a 128-row tile, from the in-kernel metadata).
// Per subchannel both operands are staged in LDS as E4M3 codes; each wave
// multiplies a 64x64 sub-tile with 16 v_mfma_scale_f32_16x16x128_f8f6f4
// (neutral E8M0 scales: the products are exact), and folds each 16x16
// partial into the fp32 accumulator with one FMA per element:
// acc += p * (sl[row] * sr).  Rows outside the item's range are zero codes in
// LDS and are never stored.
#include "gmm_device.hpp"
#include "gmm_launch.hpp"

namespace gmm {

namespace {

constexpr int kTM = 128, kTN = 128, kTK = 128;
constexpr int kPad = 16;  // LDS row padding (bytes): 144-byte rows are bank-conflict free for
                          // the 16-lane ds_read_b128 pattern below

enum LhsKind { kLhsE4M3 = 0, kLhsBF16 = 1, kLhsF32 = 2 };

// Quantise 64 consecutive K-elements of one row (this thread's half of a
// 128-wide subchannel; the partner half is in lane ^ 1) into 64 codes.
template <int KIND>
__device__ __forceinline__ float quantize_half_row(const void* __restrict__ lhs, int64_t elem,
                                                   bool valid, uint4 (&codes)[4]) {
    float v[64];
    if (valid) {
        if constexpr (KIND == kLhsBF16) {
            const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(lhs) + elem);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint4 d = p[c];
                v[8 * c + 0] = bf16_lo(d.x); v[8 * c + 1] = bf16_hi(d.x);
                v[8 * c + 2] = bf16_lo(d.y); v[8 * c + 3] = bf16_hi(d.y);
                v[8 * c + 4] = bf16_lo(d.z); v[8 * c + 5] = bf16_hi(d.z);
                v[8 * c + 6] = bf16_lo(d.w); v[8 * c + 7] = bf16_hi(d.w);
            }
        } else {
            const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(lhs) + elem);
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float4 d = p[c];
                v[4 * c + 0] = d.x; v[4 * c + 1] = d.y; v[4 * c + 2] = d.z; v[4 * c + 3] = d.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 64; ++i) v[i] = 0.0f;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    const float s = quant_scale(a);
    const float inv = quant_inv(s);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        codes[c].x = e4m3x4(v[16 * c + 0] * inv, v[16 * c + 1] * inv, v[16 * c + 2] * inv, v[16 * c + 3] * inv);
        codes[c].y = e4m3x4(v[16 * c + 4] * inv, v[16 * c + 5] * inv, v[16 * c + 6] * inv, v[16 * c + 7] * inv);
        codes[c].z = e4m3x4(v[16 * c + 8] * inv, v[16 * c + 9] * inv, v[16 * c + 10] * inv, v[16 * c + 11] * inv);
        codes[c].w = e4m3x4(v[16 * c + 12] * inv, v[16 * c + 13] * inv, v[16 * c + 14] * inv, v[16 * c + 15] * inv);
    }
    return s;
}

template <int KIND, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void fp8_fwd_kernel(
    const void* __restrict__ lhs, const float* __restrict__ lhs_scale,
    const uint8_t* __restrict__ rhs, const float* __restrict__ rhs_scale,
    const int32_t* __restrict__ group_sizes, int M, int K, int N, int G, void* __restrict__ out,
    uint8_t* __restrict__ q_out, float* __restrict__ s_out, int ntiles_n, int nblocks) {
    __shared__ WorkItem s_item;
    __shared__ __attribute__((aligned(16))) uint8_t sA[kTM][kTK + kPad];
    __shared__ __attribute__((aligned(16))) uint8_t sB[kTN][kTK + kPad];
    __shared__ float sSl[kTM];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int L = xcd_remap(blockIdx.x, nblocks);
    const int w = L / ntiles_n, nt = L % ntiles_n;
    if (wave == 0) {
        const WorkItem it = find_work_item(group_sizes, G, M, 7, w);
        if (lane == 0) s_item = it;
    }
    __syncthreads();
    const WorkItem it = s_item;
    if (it.g < 0) return;
    const int n0 = nt * kTN;

    if (it.g == G) {  // rows past the last group: zeros
        const int rows = it.hi - it.lo;
        for (int e = tid; e < rows * (kTN / 8); e += 256) {
            const int r = it.lo + e / (kTN / 8), c = n0 + (e % (kTN / 8)) * 8;
            if constexpr (OUT_BF16)
                *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + (int64_t)r * N + c) = make_uint4(0, 0, 0, 0);
            else {
                float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (int64_t)r * N + c);
                p[0] = make_float4(0, 0, 0, 0);
                p[1] = make_float4(0, 0, 0, 0);
            }
        }
        return;
    }

    const int g = it.g, row0 = it.tile * kTM;
    const int nkb = K / kQBlock, nnb = N / kQBlock;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lk = (lane >> 4) * 32;

    // staging roles: thread -> (row or column, K half)
    const int st_r = tid >> 1, st_h = tid & 1;
    const int a_row = row0 + st_r;
    const bool a_valid = a_row >= it.lo && a_row < it.hi;
    const bool write_q = q_out != nullptr && nt == 0 && a_valid;
    const uint8_t* b_src = rhs + ((int64_t)g * N + n0 + st_r) * K + st_h * 64;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb < nkb; ++kb) {
        // ---- stage A (quantise or copy codes) and B codes into LDS
        uint4 ac[4];
        float sl;
        if constexpr (KIND == kLhsE4M3) {
            if (a_valid) {
                const uint4* p = reinterpret_cast<const uint4*>(
                    reinterpret_cast<const uint8_t*>(lhs) + (int64_t)a_row * K + kb * kTK + st_h * 64);
#pragma unroll
                for (int c = 0; c < 4; ++c) ac[c] = p[c];
                sl = lhs_scale[(int64_t)a_row * nkb + kb];
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) ac[c] = make_uint4(0, 0, 0, 0);
                sl = 0.0f;
            }
        } else {
            sl = quantize_half_row<KIND>(lhs, (int64_t)a_row * K + kb * kTK + st_h * 64, a_valid, ac);
            if (write_q) {
                uint4* p = reinterpret_cast<uint4*>(q_out + (int64_t)a_row * K + kb * kTK + st_h * 64);
#pragma unroll
                for (int c = 0; c < 4; ++c) p[c] = ac[c];
                if (st_h == 0) s_out[(int64_t)a_row * nkb + kb] = sl;
            }
        }
        uint4 bc[4];
        {
            const uint4* p = reinterpret_cast<const uint4*>(b_src + kb * kTK);
#pragma unroll
            for (int c = 0; c < 4; ++c) bc[c] = p[c];
        }
        const float sr = rhs_scale[((int64_t)g * nkb + kb) * nnb + n0 / kQBlock];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            *reinterpret_cast<uint4*>(&sA[st_r][st_h * 64 + 16 * c]) = ac[c];
            *reinterpret_cast<uint4*>(&sB[st_r][st_h * 64 + 16 * c]) = bc[c];
        }
        if (st_h == 0) sSl[st_r] = sl;
        __syncthreads();

        // ---- MFMA: 4x4 blocks of 16x16, K = 128 each
        v8i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const v8i*>(&sA[wm * 64 + i * 16 + lr][lk]);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const v8i*>(&sB[wn * 64 + j * 16 + lr][lk]);
        float cs[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) cs[i][r] = sSl[wm * 64 + i * 16 + (lane >> 4) * 4 + r] * sr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], cs[i][r], acc[i][j][r]);
            }
        __syncthreads();
    }

    // ---- epilogue: masked stores of the item's rows
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
            if (row < it.lo || row >= it.hi) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 64 + j * 16 + lr;
                if constexpr (OUT_BF16)
                    reinterpret_cast<uint16_t*>(out)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
                else
                    reinterpret_cast<float*>(out)[(int64_t)row * N + col] = acc[i][j][r];
            }
        }
}

template <int KIND>
hipError_t launch_kind(const void* lhs, const float* lhs_scale, const uint8_t* rhs,
                       const float* rhs_scale, const int32_t* group_sizes, int M, int K, int N,
                       int G, void* out, bool out_bf16, uint8_t* q_out, float* scale_out,
                       hipStream_t stream) {
    const int ntiles_n = N / kTN;
    const int64_t items = max_work_items(M, G, kTM);
    const int nblocks = (int)(items * ntiles_n);
    if (out_bf16)
        hipLaunchKernelGGL((fp8_fwd_kernel<KIND, true>), dim3(nblocks), dim3(256), 0, stream, lhs,
                           lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out, q_out,
                           scale_out, ntiles_n, nblocks);
    else
        hipLaunchKernelGGL((fp8_fwd_kernel<KIND, false>), dim3(nblocks), dim3(256), 0, stream, lhs,
                           lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out, q_out,
                           scale_out, ntiles_n, nblocks);
    return hipGetLastError();
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
