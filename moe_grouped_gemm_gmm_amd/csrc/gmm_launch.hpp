// Internal launchers behind the C ABI of gmm.h.  Arguments are already
// validated by gmm_api.cpp; each launcher only enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmm_config.hpp"

namespace gmm {

// Compute units of the current device (queried once).
inline int device_cus() {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

// Every grouped launcher takes `status`: a device int32 that block 0 of the
// launch sets to the call's device status (bits kDevSumGtM, kDevNegativeSize
// of gmm_device.hpp; 0 when group_sizes keeps the contract).

// Bytes of the library-owned device scratch behind gmm_fp8_fwd_noalloc, and
// its device address on the current device (found once per device).
constexpr size_t kNoallocScratchBytes = 4096;
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Streaming read of `bytes` (a multiple of 64 KB) with one 64 KB slice per
// workgroup; sink has one word per slice.
hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                                    hipStream_t stream);

hipError_t launch_group_metadata(const int32_t* group_sizes, int G, int M, int tm,
                                 int32_t* offsets, int32_t* work, int capacity,
                                 int32_t* num_work, int32_t* status, hipStream_t stream);

// x_bf16: true for bf16 input, false for fp32.
hipError_t launch_quantize_lhs(const void* x, bool x_bf16, int64_t M, int64_t K, uint8_t* q,
                               float* scale, hipStream_t stream);

hipError_t launch_quantize_rhs(const void* w, bool w_bf16, int64_t G, int64_t K, int64_t N,
                               uint8_t* q, float* scale, hipStream_t stream);

// Logical [G,K,N] E4M3 codes into the packed order of launch_quantize_rhs.
hipError_t launch_pack_rhs(const uint8_t* q, int64_t G, int64_t K, int64_t N, uint8_t* packed,
                           hipStream_t stream);

// s = a/448 and its guarded inverse for n block abs-maxima (the quantisers'
// own device routines).
hipError_t launch_quant_scales(const float* amax, int64_t n, float* scale, float* inv,
                               hipStream_t stream);

// MXFP4 weights in the forward's packed operand order (codes G*K*N/2 bytes,
// E8M0 scales G*K*N/32 bytes).
hipError_t launch_quantize_rhs_mxfp4(const void* w, bool w_bf16, int64_t G, int64_t K, int64_t N,
                                     uint8_t* q, uint8_t* scale, hipStream_t stream);

// int4 weights (codes in [-8, 7], 128x128 fp32 block scales s = a/7) in the
// forward's packed operand order (G*K*N/2 bytes); and int4 codes made
// elsewhere (int8 values, logical [G,K,N]) into that order.
hipError_t launch_quantize_rhs_int4(const void* w, bool w_bf16, int64_t G, int64_t K, int64_t N,
                                    uint8_t* q, float* scale, hipStream_t stream);
hipError_t launch_pack_rhs_int4(const int8_t* q, int64_t G, int64_t K, int64_t N, uint8_t* packed,
                                hipStream_t stream);

// lhs_kind: 0 = E4M3 codes + lhs_scale, 1 = bf16, 2 = fp32.
hipError_t launch_fp8_fwd(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                          const uint8_t* rhs, const float* rhs_scale,
                          const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                          bool out_bf16, uint8_t* q_out, float* scale_out, int32_t* status, hipStream_t stream);

// Fused gate+up: rhs has 2N columns (gate, then up); out = silu(gate) * up,
// [M,N]; act_q/act_scale (both or neither) the 1x128 quantised activation.
hipError_t launch_fp8_fwd_swiglu(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                                 const uint8_t* rhs, const float* rhs_scale,
                                 const int32_t* group_sizes, int M, int K, int N, int G,
                                 void* out, bool out_bf16, uint8_t* act_q, float* act_scale,
                                 int32_t* status, hipStream_t stream);

// FP8 (1x128) LHS against packed MXFP4 weights.
hipError_t launch_fp8_mxfp4_fwd(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                                const uint8_t* rhs_q, const uint8_t* rhs_scale,
                                const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                                bool out_bf16, int32_t* status, hipStream_t stream);

// FP8 (1x128) LHS against packed int4 weights with 128x128 fp32 block scales.
hipError_t launch_fp8_int4_fwd(const TileConfig& cfg, const void* lhs, int lhs_kind, const float* lhs_scale,
                               const uint8_t* rhs_q, const float* rhs_scale,
                               const int32_t* group_sizes, int M, int K, int N, int G, void* out,
                               bool out_bf16, int32_t* status, hipStream_t stream);

hipError_t launch_bf16_fwd(const TileConfig& cfg, const void* lhs, const void* rhs, const int32_t* group_sizes, int M,
                           int K, int N, int G, void* out, bool out_bf16, int32_t* status, hipStream_t stream);

hipError_t launch_bf16_dx(const TileConfig& cfg, const void* dy, const void* w, const int32_t* group_sizes, int M,
                          int K, int N, int G, void* dx, bool out_bf16, int32_t* status, hipStream_t stream);

hipError_t launch_tgmm(const TileConfig& cfg, const void* x, const void* dy, const int32_t* group_sizes, int M, int K,
                       int N, int G, void* dw, bool out_bf16, int32_t* status, hipStream_t stream);

}  // namespace gmm
