// Blockwise FP8 quantisation kernels and the group-metadata exposer.
//
// LHS: one scale per row per 128 K-elements, computed from the data on every
// call; RHS: one scale per 128x128 block, computed once offline
// ("GEMM Kernel 性能优化十问", Q2).  The recipe (abs-max, s = a/448, guarded
// inverse, x*inv cast to E4M3) follows "实现差距：GMM Kernel（V1 vs V2）",
// section 3.3.
#include "gmm_device.hpp"
#include "gmm_launch.hpp"

namespace gmm {

// ------------------------------------------------------------ metadata --

__global__ __launch_bounds__(256) void group_metadata_kernel(const int32_t* __restrict__ group_sizes,
                                                             int G, int M, int tm,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ work,
                                                             int capacity,
                                                             int32_t* __restrict__ num_work,
                                                             int32_t* __restrict__ status) {
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int w = blockIdx.x * 4 + wave;
    if (w < capacity) {
        const WorkItem it = find_work_item(group_sizes, G, M, tm, w);
        if (lane == 0) {
            work[4 * w + 0] = it.g;
            work[4 * w + 1] = it.g < 0 ? 0 : it.tile;
            work[4 * w + 2] = it.g < 0 ? 0 : it.lo;
            work[4 * w + 3] = it.g < 0 ? 0 : it.hi;
        }
    }
    if (blockIdx.x == 0 && wave == 0) {
        // offsets: the first row of each group's clamped range, then the
        // clamped total; the item count: the groups' tiles plus the tail's
        int carry_rows = 0, carry_items = 0;
        bool negative = false;
        for (int base = 0; base < G; base += 64) {
            const GroupChunk ch = group_chunk(group_sizes, G, M, base, carry_rows);
            const int c = ch.hi > ch.lo ? (ch.hi - 1) / tm - ch.lo / tm + 1 : 0;
            if (base + lane < G) offsets[base + lane] = ch.lo;
            carry_rows = ch.next_carry;
            carry_items += lane_value(wave_incl_scan(c), 63);
            negative = negative || ch.negative;
        }
        if (lane == 0) {
            const int total = min(carry_rows, M);
            const int tail = total < M ? (M + tm - 1) / tm - total / tm : 0;
            offsets[G] = total;
            num_work[0] = carry_items + tail;
            status[0] = (carry_rows > M ? kDevSumGtM : 0) | (negative ? kDevNegativeSize : 0);
        }
    }
}

hipError_t launch_group_metadata(const int32_t* group_sizes, int G, int M, int tm,
                                 int32_t* offsets, int32_t* work, int capacity,
                                 int32_t* num_work, int32_t* status, hipStream_t stream) {
    const int blocks = (capacity + 3) / 4;
    hipLaunchKernelGGL(group_metadata_kernel, dim3(blocks), dim3(256), 0, stream, group_sizes, G,
                       M, tm, offsets, work, capacity, num_work, status);
    return hipGetLastError();
}

// ------------------------------------------------------------ LHS 1x128 --
// 16 lanes own one 128-element block (8 elements each, one 16-byte load for
// bf16); the abs-max is reduced across those 16 lanes.  Each lane works on
// kUnroll blocks at once to keep several loads in flight (HBM-bound pass).

constexpr int kQuantUnroll = 4;

template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t elem, float (&v)[8]) {
    if constexpr (BF16) {
        const uint4 d = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + elem);
        v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
        v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
        v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
        v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
    } else {
        const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + elem);
        const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + elem + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_lhs_kernel(const void* __restrict__ x,
                                                           int64_t nblk, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
    const int sub = threadIdx.x & 15;
    const int64_t group = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int64_t stride = (int64_t)gridDim.x * 16;
    for (int64_t b0 = group; b0 < nblk; b0 += stride * kQuantUnroll) {
        float v[kQuantUnroll][8];
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t blk = b0 + u * stride;
            if (blk < nblk) {
                load8<BF16>(x, blk * kQBlock + sub * 8, v[u]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t blk = b0 + u * stride;
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[u][i]));
            a = max_over_16(a);
            const float s = quant_scale(a);
            const float inv = quant_inv(s);
            uint2 codes;
            codes.x = e4m3x4(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv);
            codes.y = e4m3x4(v[u][4] * inv, v[u][5] * inv, v[u][6] * inv, v[u][7] * inv);
            if (blk < nblk) {
                store_out(q + blk * kQBlock + sub * 8, codes);
                if (sub == 0) store_out(&scale[blk], s);
            }
        }
    }
}

hipError_t launch_quantize_lhs(const void* x, bool x_bf16, int64_t M, int64_t K, uint8_t* q,
                               float* scale, hipStream_t stream) {
    const int64_t nblk = M * (K / kQBlock);
    int64_t blocks = (nblk + 16 * kQuantUnroll - 1) / (16 * kQuantUnroll);
    if (blocks > 4096) blocks = 4096;
    if (x_bf16)
        hipLaunchKernelGGL(quantize_lhs_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           x, nblk, q, scale);
    else
        hipLaunchKernelGGL(quantize_lhs_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           x, nblk, q, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------- RHS 128x128 --
// One workgroup per (g, kb, nb) block.  Thread t owns column n = nb*128 +
// t % 128 and the 64 K-rows of half t / 128.  The codes are written in the
// MFMA operand order gmm_fp8_fwd loads (see rhs_packed_offset): each 16-column
// by 128-K slab is 2 KB, and the 32 K-values one lane of the MFMA needs for
// one column sit as two 16-byte runs, so the forward reads whole contiguous
// kilobytes.

// Byte offset of the 16-byte run holding codes k0 .. k0+15 (k0 % 16 == 0) of
// column n in the packed RHS: [G][N/16][K/128][2][64][16], with lane
// l = 16 * ((k % 128) / 32) + n % 16 and half h = (k % 32) / 16.
__device__ __forceinline__ int64_t rhs_packed_offset(int g, int n, int k0, int N, int K) {
    const int nb16 = n >> 4, lr = n & 15, kb = k0 >> 7, lc = (k0 & 127) >> 5, h = (k0 & 31) >> 4;
    return ((((int64_t)g * (N >> 4) + nb16) * (K >> 7) + kb) * 2 + h) * 1024 + (lc * 16 + lr) * 16;
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_rhs_kernel(const void* __restrict__ w, int K,
                                                           int N, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
    __shared__ float wave_max[4];
    const int nkb = K / kQBlock, nnb = N / kQBlock;
    const int blk = blockIdx.x;
    const int g = blk / (nkb * nnb), kb = (blk / nnb) % nkb, nb = blk % nnb;
    const int t = threadIdx.x, n = nb * kQBlock + (t & 127), k0 = kb * kQBlock + (t >> 7) * 64;
    float v[64];
    const int64_t base = ((int64_t)g * K + k0) * N + n;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        if constexpr (BF16)
            v[i] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w)[base + (int64_t)i * N] << 16);
        else
            v[i] = reinterpret_cast<const float*>(w)[base + (int64_t)i * N];
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) a = fmaxf(a, __shfl_xor(a, d, 64));
    if (lane_id() == 0) wave_max[t >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const float s = quant_scale(a);
    const float inv = quant_inv(s);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        uint4 o;
        o.x = e4m3x4(v[16 * c + 0] * inv, v[16 * c + 1] * inv, v[16 * c + 2] * inv, v[16 * c + 3] * inv);
        o.y = e4m3x4(v[16 * c + 4] * inv, v[16 * c + 5] * inv, v[16 * c + 6] * inv, v[16 * c + 7] * inv);
        o.z = e4m3x4(v[16 * c + 8] * inv, v[16 * c + 9] * inv, v[16 * c + 10] * inv, v[16 * c + 11] * inv);
        o.w = e4m3x4(v[16 * c + 12] * inv, v[16 * c + 13] * inv, v[16 * c + 14] * inv, v[16 * c + 15] * inv);
        *reinterpret_cast<uint4*>(q + rhs_packed_offset(g, n, k0 + 16 * c, N, K)) = o;
    }
    if (t == 0) scale[blk] = s;
}

// ------------------------------------------------------ RHS code packing --
// E4M3 codes quantised elsewhere, logical [G,K,N], into the packed order
// above.  One workgroup per 2 KB slab (expert g, 16-column block, 128-K
// step): thread t reads the 16 codes of row k = 128*kb + t for the slab's
// columns into LDS, then writes one 16-byte run: half h = t / 64, lane
// l = t % 64 holds column 16*nb + l%16, k = 128*kb + 32*(l/16) + 16*h + e.
__global__ __launch_bounds__(128) void pack_rhs_kernel(const uint8_t* __restrict__ q, int K, int N,
                                                       uint8_t* __restrict__ packed) {
    __shared__ uint8_t tile[kQBlock][16 + 4];   // [k][n]; 20-byte rows spread the column reads
    const int nkb = K / kQBlock, nn16 = N / 16;
    const int64_t slab = blockIdx.x;               // (g * N/16 + nb) * K/128 + kb
    const int kb = (int)(slab % nkb);
    const int64_t gnb = slab / nkb;
    const int nb = (int)(gnb % nn16);
    const int64_t g = gnb / nn16;
    const int t = threadIdx.x;
    const uint4 row = *reinterpret_cast<const uint4*>(q + (g * K + kb * kQBlock + t) * N + nb * 16);
    const uint32_t words[4] = {row.x, row.y, row.z, row.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(&tile[t][4 * i]) = words[i];
    __syncthreads();
    const int h = t >> 6, l = t & 63, col = l & 15, k0 = 32 * (l >> 4) + 16 * h;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = (uint32_t)tile[k0 + 4 * i][col] | ((uint32_t)tile[k0 + 4 * i + 1][col] << 8) |
               ((uint32_t)tile[k0 + 4 * i + 2][col] << 16) | ((uint32_t)tile[k0 + 4 * i + 3][col] << 24);
    *reinterpret_cast<uint4*>(packed + slab * 2048 + h * 1024 + l * 16) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_pack_rhs(const uint8_t* q, int64_t G, int64_t K, int64_t N, uint8_t* packed,
                           hipStream_t stream) {
    const int64_t slabs = G * (N / 16) * (K / kQBlock);
    hipLaunchKernelGGL(pack_rhs_kernel, dim3((unsigned)slabs), dim3(128), 0, stream, q, (int)K,
                       (int)N, packed);
    return hipGetLastError();
}

// ------------------------------------------------------- int4 weights --
// int4 codes ("实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1 name
// int4 among the sub-byte RHS types) with the FP8 path's 128x128 blocks and
// fp32 scales; the packed order is the FP8 one at half the bytes: per
// (expert g, 16-column block, 128-K step) a 1 KB slab [64 lanes][16 bytes],
// lane l = 16 * ((k % 128) / 32) + n % 16 holding the 32 codes of column n
// and rows 128 kb + 32 (l / 16) + j, two per byte: dword d, byte i holds row
// j = 8d + i in its low nibble and row 8d + 4 + i in its high nibble, so
// that expanding a dword's low and then high nibbles gives the E4M3 operand
// bytes of rows 8d .. 8d+7 in order (int4_to_e4m3x4).

// Byte offset of the 16-byte run of column n, rows k0 .. k0+31 (k0 % 32 == 0).
__device__ __forceinline__ int64_t int4_packed_offset(int g, int n, int k0, int N, int K) {
    const int nb16 = n >> 4, lr = n & 15, kb = k0 >> 7, lc = (k0 & 127) >> 5;
    return ((((int64_t)g * (N >> 4) + nb16) * (K >> 7) + kb) * 64 + lc * 16 + lr) * 16;
}

// 32 codes of one run (c[j], rows j = 0..31) -> the run's 16 bytes.
__device__ __forceinline__ uint4 int4_run(const int* c) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v |= ((uint32_t)(c[8 * q + i] & 15) | ((uint32_t)(c[8 * q + 4 + i] & 15) << 4)) << (8 * i);
        d[q] = v;
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// One workgroup per (g, kb, nb) 128x128 block; thread t owns column
// nb*128 + t % 128 and the 64 rows of half t / 128 (two 32-row runs).
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_rhs_int4_kernel(const void* __restrict__ w, int K, int N,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
    __shared__ float wave_max[4];
    const int nkb = K / kQBlock, nnb = N / kQBlock;
    const int blk = blockIdx.x;
    const int g = blk / (nkb * nnb), kb = (blk / nnb) % nkb, nb = blk % nnb;
    const int t = threadIdx.x, n = nb * kQBlock + (t & 127), k0 = kb * kQBlock + (t >> 7) * 64;
    float v[64];
    const int64_t base = ((int64_t)g * K + k0) * N + n;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        if constexpr (BF16)
            v[i] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w)[base + (int64_t)i * N] << 16);
        else
            v[i] = reinterpret_cast<const float*>(w)[base + (int64_t)i * N];
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) a = fmaxf(a, __shfl_xor(a, d, 64));
    if (lane_id() == 0) wave_max[t >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const float s = quant_scale7(a);
    const float inv = quant_inv(s);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        int c[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) c[j] = int4_code(v[32 * r + j], inv);
        *reinterpret_cast<uint4*>(q + int4_packed_offset(g, n, k0 + 32 * r, N, K)) = int4_run(c);
    }
    if (t == 0) scale[blk] = s;
}

// int4 codes made elsewhere (int8 values in [-8, 7], logical [G,K,N]) into the
// packed order.  One workgroup per 1 KB slab: 128 threads stage the slab's
// 128 rows x 16 columns in LDS, then 64 of them write one 16-byte run each.
__global__ __launch_bounds__(128) void pack_rhs_int4_kernel(const int8_t* __restrict__ q, int K, int N,
                                                            uint8_t* __restrict__ packed) {
    __shared__ int8_t tile[kQBlock][16 + 4];
    const int nkb = K / kQBlock, nn16 = N / 16;
    const int64_t slab = blockIdx.x;               // (g * N/16 + nb) * K/128 + kb
    const int kb = (int)(slab % nkb);
    const int64_t gnb = slab / nkb;
    const int nb = (int)(gnb % nn16);
    const int64_t g = gnb / nn16;
    const int t = threadIdx.x;
    const uint4 row = *reinterpret_cast<const uint4*>(q + (g * K + kb * kQBlock + t) * N + nb * 16);
    const uint32_t words[4] = {row.x, row.y, row.z, row.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(&tile[t][4 * i]) = words[i];
    __syncthreads();
    if (t >= 64) return;
    const int col = t & 15, j0 = 32 * (t >> 4);
    int c[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = tile[j0 + j][col];
    *reinterpret_cast<uint4*>(packed + slab * 1024 + t * 16) = int4_run(c);
}

hipError_t launch_quantize_rhs_int4(const void* w, bool bf16, int64_t G, int64_t K, int64_t N, uint8_t* q,
                                    float* scale, hipStream_t stream) {
    const int64_t blocks = G * (K / kQBlock) * (N / kQBlock);
    if (bf16)
        hipLaunchKernelGGL(quantize_rhs_int4_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                           (int)K, (int)N, q, scale);
    else
        hipLaunchKernelGGL(quantize_rhs_int4_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                           (int)K, (int)N, q, scale);
    return hipGetLastError();
}

hipError_t launch_pack_rhs_int4(const int8_t* q, int64_t G, int64_t K, int64_t N, uint8_t* packed,
                                hipStream_t stream) {
    const int64_t slabs = G * (N / 16) * (K / kQBlock);
    hipLaunchKernelGGL(pack_rhs_int4_kernel, dim3((unsigned)slabs), dim3(128), 0, stream, q, (int)K,
                       (int)N, packed);
    return hipGetLastError();
}

// ---------------------------------------------- the recipe's scale pair --
// s = a/448 and inv = (s == 0 ? 0 : 1/s) for a list of block abs-maxima,
// through the same device routines every quantiser above and the fused
// forward use (quant_scale, quant_inv).
__global__ __launch_bounds__(256) void quant_scales_kernel(const float* __restrict__ amax, int64_t n,
                                                           float* __restrict__ scale,
                                                           float* __restrict__ inv) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const float s = quant_scale(amax[i]);
        scale[i] = s;
        inv[i] = quant_inv(s);
    }
}

hipError_t launch_quant_scales(const float* amax, int64_t n, float* scale, float* inv,
                               hipStream_t stream) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(quant_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, amax, n,
                       scale, inv);
    return hipGetLastError();
}

// --------------------------------------------------------- MXFP4 RHS --
//
// "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1: RHS weights in a
// sub-byte type, MXFP4 first.  Format and conversion follow the OCP MX
// specification v1.0: blocks of 32 consecutive k of one (expert, column)
// share an E8M0 scale 2^(e-127) with e = floor(log2(max|w|)) - 2, clamped to
// [-127, 127] (code 0 for an all-zero block); each element becomes the E2M1
// value nearest to w / 2^e (ties to the even mantissa, clamped to +-6,
// sign kept).
//
// Packed layout, the operand order of the forward's MFMA: per (expert g,
// 16-column block, 128-K step) a 1 KB chunk of codes and a 64-byte chunk of
// scales, chunk index c = (g * N/16 + n/16) * K/128 + k/128.  Lane
// l = 16 * swap2((k % 128) / 32) + n % 16 (swap2 exchanges the two bits of a
// 2-bit index) owns bytes c*1024 + 16l .. +15, holding the 32 codes of its
// MX block in k order, two per byte, even k in the low nibble; scale byte
// c*64 + l is that block's E8M0 code.  (With an FP4 first operand the MFMA
// groups K so that lane group q pairs with K positions 64(q%2) + 16(q/2) +
// {0..15, 32..47}; the forward stores the LHS with K runs 1<->2 and 5<->6 of
// 16 exchanged, which makes lane group q's positions hold MX block swap2(q)
// contiguously.)

__device__ __forceinline__ int swap2(int q) { return ((q & 1) << 1) | (q >> 1); }

__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const float a = fabsf(y);
    const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                       (a >= 3.5f) + (a > 5.0f);
    return c | (signbit(y) ? 8u : 0u);
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_rhs_mxfp4_kernel(const void* __restrict__ w, int K,
                                                                 int N, uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ scale) {
    const int nkb = K / kQBlock, nb64 = N / 64;
    const int blk = blockIdx.x;
    const int g = blk / (nkb * nb64), kb = (blk / nb64) % nkb, nbl = blk % nb64;
    const int t = threadIdx.x, n = nbl * 64 + (t & 63), sub = t >> 6;
    const int64_t base = ((int64_t)g * K + kb * kQBlock + sub * 32) * N + n;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if constexpr (BF16)
            v[i] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w)[base + (int64_t)i * N] << 16);
        else
            v[i] = reinterpret_cast<const float*>(w)[base + (int64_t)i * N];
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    uint32_t e8 = 0;
    if (a > 0.0f) {
        int ex;
        frexpf(a, &ex);                       // a = f 2^ex, f in [0.5, 1)
        const int e = min(max(ex - 1 - 2, -127), 127);
#pragma unroll
        for (int i = 0; i < 32; ++i) words[i / 8] |= e2m1_code(ldexpf(v[i], -e)) << (4 * (i % 8));
        e8 = (uint32_t)(e + 127);
    }
    const int64_t chunk = ((int64_t)g * (N / 16) + n / 16) * nkb + kb;
    const int lane = 16 * swap2(sub) + (n & 15);
    *reinterpret_cast<uint4*>(q + chunk * 1024 + lane * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    scale[chunk * 64 + lane] = (uint8_t)e8;
}

hipError_t launch_quantize_rhs_mxfp4(const void* w, bool w_bf16, int64_t G, int64_t K, int64_t N,
                                     uint8_t* q, uint8_t* scale, hipStream_t stream) {
    const int64_t blocks = G * (K / kQBlock) * (N / 64);
    if (w_bf16)
        hipLaunchKernelGGL(quantize_rhs_mxfp4_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, w, (int)K, (int)N, q, scale);
    else
        hipLaunchKernelGGL(quantize_rhs_mxfp4_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, w, (int)K, (int)N, q, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_rhs(const void* w, bool w_bf16, int64_t G, int64_t K, int64_t N,
                               uint8_t* q, float* scale, hipStream_t stream) {
    const int64_t blocks = G * (K / kQBlock) * (N / kQBlock);
    if (w_bf16)
        hipLaunchKernelGGL(quantize_rhs_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           w, (int)K, (int)N, q, scale);
    else
        hipLaunchKernelGGL(quantize_rhs_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           w, (int)K, (int)N, q, scale);
    return hipGetLastError();
}

}  // namespace gmm
