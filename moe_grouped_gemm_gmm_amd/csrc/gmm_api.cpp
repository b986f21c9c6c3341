// C ABI of the grouped-matmul library (declared in include/gmm.h): host-side
// argument checks, then one launch on the caller's stream.  Nothing here
// allocates; only gmm_device_status synchronises (it reads one word of a
// workspace back to the host).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "../../include/gmm.h"
#include "gmm_config.hpp"
#include "gmm_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1024;

int check_ptr(const void* p, const char* name) {
    if (p == nullptr) return fail(GMM_ERR_NULL, "%s is NULL", name);
    if (!aligned16(p)) return fail(GMM_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return GMM_OK;
}

int check_opt_ptr(const void* p, const char* name) {
    if (p != nullptr && !aligned16(p)) return fail(GMM_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return GMM_OK;
}

int check_groups(int64_t M, int64_t G) {
    if (M < 0 || M > kMaxDim) return fail(GMM_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (G < 1 || G > GMM_MAX_GROUPS)
        return fail(GMM_ERR_SHAPE, "G=%lld outside [1, %d]", (long long)G, GMM_MAX_GROUPS);
    return GMM_OK;
}

int check_mult(int64_t v, int64_t mult, const char* name) {
    if (v < mult || v > kMaxDim || v % mult != 0)
        return fail(GMM_ERR_SHAPE, "%s=%lld must be a positive multiple of %lld", name,
                    (long long)v, (long long)mult);
    return GMM_OK;
}

int check_out_dtype(int dt, const char* name) {
    if (dt != GMM_BF16 && dt != GMM_F32)
        return fail(GMM_ERR_DTYPE, "%s dtype %d is not GMM_BF16 or GMM_F32", name, dt);
    return GMM_OK;
}

// Bytes of the status block at the start of every workspace (word 0: the
// device status of the last call that used it).
constexpr size_t kWsStatusBytes = 256;

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (ws == nullptr || ws_bytes < need)
        return fail(GMM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed%s", ws == nullptr ? 0 : ws_bytes,
                    need, ws == nullptr ? " (ws is NULL)" : "");
    if (!aligned16(ws)) return fail(GMM_ERR_ALIGN, "ws is not 16-byte aligned");
    return GMM_OK;
}

int32_t* ws_status(void* ws) { return reinterpret_cast<int32_t*>(ws); }

// The tile configuration a call runs (the library's choice, or the override
// a tile search set); an override that does not fit the shape is an error.
int resolve(int op, int64_t M, int64_t K, int64_t N, int64_t G, int kind, bool out_bf16,
            bool write_q, gmm::TileConfig* cfg) {
    const char* why = "";
    if (!gmm::resolve_tile_config(op, M, K, N, G, kind, out_bf16, write_q, cfg, &why))
        return fail(GMM_ERR_SHAPE, "the tile configuration set for this operation does not fit: %s", why);
    return GMM_OK;
}

static_assert(sizeof(gmm_tile_config) == sizeof(gmm::TileConfig), "tile config layouts");

gmm::TileConfig to_internal(const gmm_tile_config& c) {
    return gmm::TileConfig{c.kernel, c.waves, c.tile_m, c.tile_n, c.depth, c.residency, c.placement};
}

gmm_tile_config to_public(const gmm::TileConfig& c) {
    gmm_tile_config o;
    o.kernel = c.kernel;
    o.waves = c.waves;
    o.tile_m = c.tile_m;
    o.tile_n = c.tile_n;
    o.depth = c.depth;
    o.residency = c.residency;
    o.placement = c.placement;
    return o;
}

int hip_status(hipError_t e) {
    if (e != hipSuccess) return fail(GMM_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return GMM_OK;
}

#define GMM_TRY(expr)                 \
    do {                              \
        int _rc = (expr);             \
        if (_rc != GMM_OK) return _rc; \
    } while (0)

}  // namespace

extern "C" {

const char* gmm_status_string(int status) {
    switch (status) {
        case GMM_OK: return "ok";
        case GMM_ERR_NULL: return "null pointer";
        case GMM_ERR_SHAPE: return "invalid shape";
        case GMM_ERR_ALIGN: return "misaligned pointer";
        case GMM_ERR_DTYPE: return "unsupported dtype";
        case GMM_ERR_WORKSPACE: return "workspace missing or too small";
        case GMM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* gmm_last_error(void) { return g_last_error; }

size_t gmm_workspace_bytes(int op, int64_t M, int64_t K, int64_t N, int64_t G) {
    (void)M; (void)K; (void)N; (void)G;
    switch (op) {
        case GMM_OP_METADATA:
        case GMM_OP_FP8_FWD:
        case GMM_OP_FP8_FWD_SWIGLU:
        case GMM_OP_FP8_MXFP4_FWD:
        case GMM_OP_BF16_FWD:
        case GMM_OP_TGMM:
        case GMM_OP_DX:
        case GMM_OP_FP8_INT4_FWD:
            return kWsStatusBytes;
        default:
            return 0;
    }
}

int gmm_set_tile_config(int op, const gmm_tile_config* cfg) {
    if (op < GMM_OP_FP8_FWD || op > GMM_OP_FP8_INT4_FWD)
        return fail(GMM_ERR_SHAPE, "op %d has no tile configuration", op);
    if (cfg == nullptr) {
        gmm::set_tile_override(op, nullptr);
        return GMM_OK;
    }
    const gmm::TileConfig c = to_internal(*cfg);
    auto in = [](int v, std::initializer_list<int> ok) {
        for (int o : ok)
            if (v == o) return true;
        return false;
    };
    if (!in(c.kernel, {0, 1, 2, 3}) || !in(c.waves, {0, 4, 8, 12, 16}) || !in(c.tile_m, {0, 48, 64}) ||
        !in(c.tile_n, {0, 128, 256, 512}) || !in(c.depth, {0, 1, 2, 3, 4}) || !in(c.residency, {0, 1, 2, 3}) ||
        !in(c.placement, {0, 1, 2}))
        return fail(GMM_ERR_SHAPE, "a tile configuration field is out of range");
    gmm::set_tile_override(op, &c);
    return GMM_OK;
}

int gmm_get_tile_config(int op, int64_t M, int64_t K, int64_t N, int64_t G, int lhs_dtype,
                        int out_dtype, gmm_tile_config* cfg) {
    if (op < GMM_OP_FP8_FWD || op > GMM_OP_FP8_INT4_FWD)
        return fail(GMM_ERR_SHAPE, "op %d has no tile configuration", op);
    if (cfg == nullptr) return fail(GMM_ERR_NULL, "cfg is NULL");
    GMM_TRY(check_out_dtype(out_dtype, "out"));
    const int kind = lhs_dtype == GMM_E4M3 ? 0 : (lhs_dtype == GMM_BF16 ? 1 : 2);
    gmm::TileConfig c;
    GMM_TRY(resolve(op, M, K, N, G, kind, out_dtype == GMM_BF16, false, &c));
    *cfg = to_public(c);
    return GMM_OK;
}

int gmm_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    constexpr int64_t kSlice = 64 * 1024;
    if (bytes < kSlice || bytes % kSlice != 0 || bytes / kSlice > kMaxDim)
        return fail(GMM_ERR_SHAPE, "bytes=%lld must be a positive multiple of 65536", (long long)bytes);
    GMM_TRY(check_ptr(buf, "buf"));
    GMM_TRY(check_ptr(sink, "sink"));
    return hip_status(gmm::launch_probe_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

int gmm_device_status(const void* ws, int32_t* status, void* stream) {
    GMM_TRY(check_ptr(ws, "ws"));
    if (status == nullptr) return fail(GMM_ERR_NULL, "status is NULL");
    hipError_t e = hipMemcpyAsync(status, ws, sizeof(int32_t), hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    return hip_status(e);
}

int gmm_pack_rhs(const uint8_t* q, int64_t G, int64_t K, int64_t N, uint8_t* packed, void* stream) {
    if (G < 1 || G > GMM_MAX_GROUPS)
        return fail(GMM_ERR_SHAPE, "G=%lld outside [1, %d]", (long long)G, GMM_MAX_GROUPS);
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    if (G * (N / 16) * (K / 128) > kMaxDim) return fail(GMM_ERR_SHAPE, "too many blocks");
    GMM_TRY(check_ptr(q, "q"));
    GMM_TRY(check_ptr(packed, "packed"));
    return hip_status(gmm::launch_pack_rhs(q, G, K, N, packed, (hipStream_t)stream));
}

int gmm_quant_scales(const float* amax, int64_t n, float* scale, float* inv, void* stream) {
    if (n < 0 || n > kMaxDim) return fail(GMM_ERR_SHAPE, "n=%lld out of range", (long long)n);
    GMM_TRY(check_ptr(amax, "amax"));
    GMM_TRY(check_ptr(scale, "scale"));
    GMM_TRY(check_ptr(inv, "inv"));
    if (n == 0) return GMM_OK;
    return hip_status(gmm::launch_quant_scales(amax, n, scale, inv, (hipStream_t)stream));
}

int gmm_group_metadata(const int32_t* group_sizes, int64_t G, int64_t M, int64_t tile_m,
                       int32_t* offsets, int32_t* work, int64_t capacity, int32_t* num_work,
                       void* ws, size_t ws_bytes, void* stream) {
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(offsets, "offsets"));
    GMM_TRY(check_ptr(work, "work"));
    GMM_TRY(check_ptr(num_work, "num_work"));
    if (tile_m < 16 || tile_m > 1024 || tile_m % 16 != 0)
        return fail(GMM_ERR_SHAPE, "tile_m=%lld is not a multiple of 16 in [16,1024]", (long long)tile_m);
    const int64_t need = (M + tile_m - 1) / tile_m + G + 1;
    if (capacity < need || capacity > kMaxDim)
        return fail(GMM_ERR_SHAPE, "capacity=%lld, need >= %lld", (long long)capacity, (long long)need);
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_METADATA, M, 0, 0, G)));
    return hip_status(gmm::launch_group_metadata(group_sizes, (int)G, (int)M, (int)tile_m, offsets,
                                                 work, (int)capacity, num_work, ws_status(ws),
                                                 (hipStream_t)stream));
}

int gmm_quantize_lhs(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* q, float* scale,
                     void* stream) {
    if (x_dtype != GMM_BF16 && x_dtype != GMM_F32)
        return fail(GMM_ERR_DTYPE, "x dtype %d is not GMM_BF16 or GMM_F32", x_dtype);
    if (M < 0 || M > kMaxDim) return fail(GMM_ERR_SHAPE, "M=%lld out of range", (long long)M);
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_ptr(x, "x"));
    GMM_TRY(check_ptr(q, "q"));
    GMM_TRY(check_ptr(scale, "scale"));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_quantize_lhs(x, x_dtype == GMM_BF16, M, K, q, scale,
                                               (hipStream_t)stream));
}

int gmm_quantize_rhs(const void* w, int w_dtype, int64_t G, int64_t K, int64_t N, uint8_t* q,
                     float* scale, void* stream) {
    if (w_dtype != GMM_BF16 && w_dtype != GMM_F32)
        return fail(GMM_ERR_DTYPE, "w dtype %d is not GMM_BF16 or GMM_F32", w_dtype);
    if (G < 1 || G > GMM_MAX_GROUPS)
        return fail(GMM_ERR_SHAPE, "G=%lld outside [1, %d]", (long long)G, GMM_MAX_GROUPS);
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    if (G * (K / 128) * (N / 128) > kMaxDim) return fail(GMM_ERR_SHAPE, "too many blocks");
    GMM_TRY(check_ptr(w, "w"));
    GMM_TRY(check_ptr(q, "q"));
    GMM_TRY(check_ptr(scale, "scale"));
    return hip_status(gmm::launch_quantize_rhs(w, w_dtype == GMM_BF16, G, K, N, q, scale,
                                               (hipStream_t)stream));
}

int gmm_quantize_rhs_mxfp4(const void* w, int w_dtype, int64_t G, int64_t K, int64_t N,
                           uint8_t* q, uint8_t* scale, void* stream) {
    if (w_dtype != GMM_BF16 && w_dtype != GMM_F32)
        return fail(GMM_ERR_DTYPE, "w dtype %d is not GMM_BF16 or GMM_F32", w_dtype);
    if (G < 1 || G > GMM_MAX_GROUPS)
        return fail(GMM_ERR_SHAPE, "G=%lld outside [1, %d]", (long long)G, GMM_MAX_GROUPS);
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    if (G * (K / 128) * (N / 64) > kMaxDim) return fail(GMM_ERR_SHAPE, "too many blocks");
    GMM_TRY(check_ptr(w, "w"));
    GMM_TRY(check_ptr(q, "q"));
    GMM_TRY(check_ptr(scale, "scale"));
    return hip_status(gmm::launch_quantize_rhs_mxfp4(w, w_dtype == GMM_BF16, G, K, N, q, scale,
                                                     (hipStream_t)stream));
}

int gmm_fp8_mxfp4_fwd(const void* lhs, int lhs_dtype, const float* lhs_scale,
                      const uint8_t* rhs_q, const uint8_t* rhs_scale, const int32_t* group_sizes,
                      int64_t M, int64_t K, int64_t N, int64_t G, void* out, int out_dtype,
                      void* ws, size_t ws_bytes, void* stream) {
    int kind;
    if (lhs_dtype == GMM_E4M3) kind = 0;
    else if (lhs_dtype == GMM_BF16) kind = 1;
    else if (lhs_dtype == GMM_F32) kind = 2;
    else return fail(GMM_ERR_DTYPE, "lhs dtype %d unsupported", lhs_dtype);
    GMM_TRY(check_out_dtype(out_dtype, "out"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    GMM_TRY(check_ptr(lhs, "lhs"));
    GMM_TRY(check_ptr(rhs_q, "rhs_q"));
    GMM_TRY(check_ptr(rhs_scale, "rhs_scale"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(out, "out"));
    if (kind == 0) GMM_TRY(check_ptr(lhs_scale, "lhs_scale"));
    else if (lhs_scale != nullptr) return fail(GMM_ERR_DTYPE, "lhs_scale given with an unquantised lhs");
    const int64_t blocks = ((M + 47) / 48 + G + 1) * (N / 128);
    if (blocks > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_FP8_MXFP4_FWD, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_FP8_MXFP4_FWD, M, K, N, G, kind, out_dtype == GMM_BF16, false, &cfg));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_fp8_mxfp4_fwd(cfg, lhs, kind, lhs_scale, rhs_q, rhs_scale, group_sizes,
                                                (int)M, (int)K, (int)N, (int)G, out,
                                                out_dtype == GMM_BF16, ws_status(ws),
                                                (hipStream_t)stream));
}

int gmm_quantize_rhs_int4(const void* w, int w_dtype, int64_t G, int64_t K, int64_t N, uint8_t* q,
                          float* scale, void* stream) {
    if (w_dtype != GMM_BF16 && w_dtype != GMM_F32)
        return fail(GMM_ERR_DTYPE, "w dtype %d is not GMM_BF16 or GMM_F32", w_dtype);
    if (G < 1 || G > GMM_MAX_GROUPS)
        return fail(GMM_ERR_SHAPE, "G=%lld outside [1, %d]", (long long)G, GMM_MAX_GROUPS);
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    if (G * (K / 128) * (N / 128) > kMaxDim) return fail(GMM_ERR_SHAPE, "too many blocks");
    GMM_TRY(check_ptr(w, "w"));
    GMM_TRY(check_ptr(q, "q"));
    GMM_TRY(check_ptr(scale, "scale"));
    return hip_status(gmm::launch_quantize_rhs_int4(w, w_dtype == GMM_BF16, G, K, N, q, scale,
                                                    (hipStream_t)stream));
}

int gmm_pack_rhs_int4(const int8_t* q, int64_t G, int64_t K, int64_t N, uint8_t* packed, void* stream) {
    if (G < 1 || G > GMM_MAX_GROUPS)
        return fail(GMM_ERR_SHAPE, "G=%lld outside [1, %d]", (long long)G, GMM_MAX_GROUPS);
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    if (G * (N / 16) * (K / 128) > kMaxDim) return fail(GMM_ERR_SHAPE, "too many slabs");
    GMM_TRY(check_ptr(q, "q"));
    GMM_TRY(check_ptr(packed, "packed"));
    const uintptr_t a = (uintptr_t)q, b = (uintptr_t)packed;
    const uintptr_t na = (uintptr_t)(G * K * N), nb = na / 2;
    if (a < b + nb && b < a + na) return fail(GMM_ERR_SHAPE, "packed overlaps q");
    return hip_status(gmm::launch_pack_rhs_int4(q, G, K, N, packed, (hipStream_t)stream));
}

int gmm_fp8_int4_fwd(const void* lhs, int lhs_dtype, const float* lhs_scale, const uint8_t* rhs_q,
                     const float* rhs_scale, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                     int64_t G, void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
    int kind;
    if (lhs_dtype == GMM_E4M3) kind = 0;
    else if (lhs_dtype == GMM_BF16) kind = 1;
    else if (lhs_dtype == GMM_F32) kind = 2;
    else return fail(GMM_ERR_DTYPE, "lhs dtype %d unsupported", lhs_dtype);
    GMM_TRY(check_out_dtype(out_dtype, "out"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    GMM_TRY(check_ptr(lhs, "lhs"));
    GMM_TRY(check_ptr(rhs_q, "rhs_q"));
    GMM_TRY(check_ptr(rhs_scale, "rhs_scale"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(out, "out"));
    if (kind == 0) GMM_TRY(check_ptr(lhs_scale, "lhs_scale"));
    else if (lhs_scale != nullptr) return fail(GMM_ERR_DTYPE, "lhs_scale given with an unquantised lhs");
    const int64_t blocks = ((M + 47) / 48 + G + 1) * (N / 128);
    if (blocks > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_FP8_INT4_FWD, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_FP8_INT4_FWD, M, K, N, G, kind, out_dtype == GMM_BF16, false, &cfg));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_fp8_int4_fwd(cfg, lhs, kind, lhs_scale, rhs_q, rhs_scale, group_sizes,
                                               (int)M, (int)K, (int)N, (int)G, out, out_dtype == GMM_BF16,
                                               ws_status(ws), (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Argument checks of gmm_fp8_fwd (and its no-allocation variant); on success
// *kind is the LHS kind of the launchers.
int check_fp8_fwd(const void* lhs, int lhs_dtype, const float* lhs_scale, const uint8_t* rhs,
                  const float* rhs_scale, const int32_t* group_sizes, int64_t M, int64_t K,
                  int64_t N, int64_t G, void* out, int out_dtype, uint8_t* q_out,
                  float* scale_out, int* kind) {
    if (lhs_dtype == GMM_E4M3) *kind = 0;
    else if (lhs_dtype == GMM_BF16) *kind = 1;
    else if (lhs_dtype == GMM_F32) *kind = 2;
    else return fail(GMM_ERR_DTYPE, "lhs dtype %d unsupported", lhs_dtype);
    GMM_TRY(check_out_dtype(out_dtype, "out"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    GMM_TRY(check_ptr(lhs, "lhs"));
    GMM_TRY(check_ptr(rhs, "rhs"));
    GMM_TRY(check_ptr(rhs_scale, "rhs_scale"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(out, "out"));
    if (*kind == 0) {
        GMM_TRY(check_ptr(lhs_scale, "lhs_scale"));
        if (q_out != nullptr || scale_out != nullptr)
            return fail(GMM_ERR_DTYPE, "q_out/scale_out need a bf16 or fp32 lhs");
    } else {
        if (lhs_scale != nullptr) return fail(GMM_ERR_DTYPE, "lhs_scale given with an unquantised lhs");
        if ((q_out == nullptr) != (scale_out == nullptr))
            return fail(GMM_ERR_NULL, "q_out and scale_out must both be set or both NULL");
        GMM_TRY(check_opt_ptr(q_out, "q_out"));
        GMM_TRY(check_opt_ptr(scale_out, "scale_out"));
    }
    const int64_t blocks = ((M + 47) / 48 + G + 1) * (N / 128);   // worst case over tile shapes
    if (blocks > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    return GMM_OK;
}

}  // namespace

extern "C" {

int gmm_fp8_fwd(const void* lhs, int lhs_dtype, const float* lhs_scale, const uint8_t* rhs,
                const float* rhs_scale, const int32_t* group_sizes, int64_t M, int64_t K,
                int64_t N, int64_t G, void* out, int out_dtype, uint8_t* q_out,
                float* scale_out, void* ws, size_t ws_bytes, void* stream) {
    int kind = 0;
    GMM_TRY(check_fp8_fwd(lhs, lhs_dtype, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                          out_dtype, q_out, scale_out, &kind));
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_FP8_FWD, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_FP8_FWD, M, K, N, G, kind, out_dtype == GMM_BF16,
                    kind != 0 && q_out != nullptr, &cfg));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_fp8_fwd(cfg, lhs, kind, lhs_scale, rhs, rhs_scale, group_sizes,
                                          (int)M, (int)K, (int)N, (int)G, out,
                                          out_dtype == GMM_BF16, q_out, scale_out, ws_status(ws),
                                          (hipStream_t)stream));
}

int gmm_fp8_fwd_noalloc(const void* lhs, int lhs_dtype, const float* lhs_scale,
                        const uint8_t* rhs, const float* rhs_scale, const int32_t* group_sizes,
                        int64_t M, int64_t K, int64_t N, int64_t G, void* out, int out_dtype,
                        uint8_t* q_out, float* scale_out, void* stream) {
    int kind = 0;
    GMM_TRY(check_fp8_fwd(lhs, lhs_dtype, lhs_scale, rhs, rhs_scale, group_sizes, M, K, N, G, out,
                          out_dtype, q_out, scale_out, &kind));
    const size_t need = gmm_workspace_bytes(GMM_OP_FP8_FWD, M, K, N, G);
    if (need > gmm::kNoallocScratchBytes)
        return fail(GMM_ERR_WORKSPACE,
                    "this shape needs %zu bytes of workspace; the library's static scratch holds %zu",
                    need, gmm::kNoallocScratchBytes);
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_FP8_FWD, M, K, N, G, kind, out_dtype == GMM_BF16,
                    kind != 0 && q_out != nullptr, &cfg));
    if (M == 0) return GMM_OK;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    GMM_TRY(hip_status(gmm::noalloc_scratch(&ws, &ws_bytes)));
    return hip_status(gmm::launch_fp8_fwd(cfg, lhs, kind, lhs_scale, rhs, rhs_scale, group_sizes,
                                          (int)M, (int)K, (int)N, (int)G, out,
                                          out_dtype == GMM_BF16, q_out, scale_out, ws_status(ws),
                                          (hipStream_t)stream));
}

int gmm_fp8_fwd_swiglu(const void* lhs, int lhs_dtype, const float* lhs_scale, const uint8_t* rhs,
                       const float* rhs_scale, const int32_t* group_sizes, int64_t M, int64_t K,
                       int64_t N, int64_t G, void* out, int out_dtype, uint8_t* act_q,
                       float* act_scale, void* ws, size_t ws_bytes, void* stream) {
    int kind;
    if (lhs_dtype == GMM_E4M3) kind = 0;
    else if (lhs_dtype == GMM_BF16) kind = 1;
    else if (lhs_dtype == GMM_F32) kind = 2;
    else return fail(GMM_ERR_DTYPE, "lhs dtype %d unsupported", lhs_dtype);
    GMM_TRY(check_out_dtype(out_dtype, "out"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 256, "N"));
    GMM_TRY(check_ptr(lhs, "lhs"));
    GMM_TRY(check_ptr(rhs, "rhs"));
    GMM_TRY(check_ptr(rhs_scale, "rhs_scale"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(out, "out"));
    if (kind == 0) GMM_TRY(check_ptr(lhs_scale, "lhs_scale"));
    else if (lhs_scale != nullptr) return fail(GMM_ERR_DTYPE, "lhs_scale given with an unquantised lhs");
    if ((act_q == nullptr) != (act_scale == nullptr))
        return fail(GMM_ERR_NULL, "act_q and act_scale must both be set or both NULL");
    GMM_TRY(check_opt_ptr(act_q, "act_q"));
    GMM_TRY(check_opt_ptr(act_scale, "act_scale"));
    const int64_t blocks = ((M + 47) / 48 + G + 1) * (N / 256);
    if (blocks > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_FP8_FWD_SWIGLU, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_FP8_FWD_SWIGLU, M, K, N, G, kind, out_dtype == GMM_BF16, false, &cfg));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_fp8_fwd_swiglu(cfg, lhs, kind, lhs_scale, rhs, rhs_scale,
                                                 group_sizes, (int)M, (int)K, (int)N, (int)G, out,
                                                 out_dtype == GMM_BF16, act_q, act_scale,
                                                 ws_status(ws), (hipStream_t)stream));
}

int gmm_bf16_fwd(const void* lhs, const void* rhs, const int32_t* group_sizes, int64_t M,
                 int64_t K, int64_t N, int64_t G, void* out, int out_dtype, void* ws,
                 size_t ws_bytes, void* stream) {
    GMM_TRY(check_out_dtype(out_dtype, "out"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 64, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    GMM_TRY(check_ptr(lhs, "lhs"));
    GMM_TRY(check_ptr(rhs, "rhs"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(out, "out"));
    const int64_t blocks = ((M + 127) / 128 + G + 1) * (N / 128);
    if (blocks > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_BF16_FWD, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_BF16_FWD, M, K, N, G, 1, out_dtype == GMM_BF16, false, &cfg));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_bf16_fwd(cfg, lhs, rhs, group_sizes, (int)M, (int)K, (int)N, (int)G,
                                           out, out_dtype == GMM_BF16, ws_status(ws),
                                           (hipStream_t)stream));
}

int tgmm_bf16(const void* x, const void* dy, const int32_t* group_sizes, int64_t M, int64_t K,
              int64_t N, int64_t G, void* dw, int out_dtype, void* ws, size_t ws_bytes,
              void* stream) {
    GMM_TRY(check_out_dtype(out_dtype, "dw"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 128, "N"));
    GMM_TRY(check_ptr(x, "x"));
    GMM_TRY(check_ptr(dy, "dy"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(dw, "dw"));
    if (G * (K / 128) * (N / 128) > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_TGMM, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_TGMM, M, K, N, G, 1, out_dtype == GMM_BF16, false, &cfg));
    return hip_status(gmm::launch_tgmm(cfg, x, dy, group_sizes, (int)M, (int)K, (int)N, (int)G, dw,
                                       out_dtype == GMM_BF16, ws_status(ws), (hipStream_t)stream));
}

int gmm_bf16_dx(const void* dy, const void* w, const int32_t* group_sizes, int64_t M, int64_t K,
                int64_t N, int64_t G, void* dx, int out_dtype, void* ws, size_t ws_bytes,
                void* stream) {
    GMM_TRY(check_out_dtype(out_dtype, "dx"));
    GMM_TRY(check_groups(M, G));
    GMM_TRY(check_mult(K, 128, "K"));
    GMM_TRY(check_mult(N, 64, "N"));
    GMM_TRY(check_ptr(dy, "dy"));
    GMM_TRY(check_ptr(w, "w"));
    GMM_TRY(check_ptr(group_sizes, "group_sizes"));
    GMM_TRY(check_ptr(dx, "dx"));
    const int64_t blocks = ((M + 127) / 128 + G + 1) * (K / 128);
    if (blocks > kMaxDim) return fail(GMM_ERR_SHAPE, "grid too large");
    GMM_TRY(check_ws(ws, ws_bytes, gmm_workspace_bytes(GMM_OP_DX, M, K, N, G)));
    gmm::TileConfig cfg;
    GMM_TRY(resolve(GMM_OP_DX, M, K, N, G, 1, out_dtype == GMM_BF16, false, &cfg));
    if (M == 0) return GMM_OK;
    return hip_status(gmm::launch_bf16_dx(cfg, dy, w, group_sizes, (int)M, (int)K, (int)N, (int)G, dx,
                                          out_dtype == GMM_BF16, ws_status(ws), (hipStream_t)stream));
}

}  // extern "C"
