// Tile configurations of the grouped kernels: the library's own choice per
// operation and shape, and a process-wide override for tile searches
// ("GEMM Kernel 性能优化十问", Q4: each phase gets its own tiling; Q8: the
// tiling is found by searching the configuration space).
#pragma once

#include <stdint.h>

namespace gmm {

// Operation ids (the gmm_op values of gmm.h).
enum Op { kOpMetadata = 0, kOpFp8Fwd = 1, kOpFp8Swiglu = 2, kOpFp8Mxfp4 = 3, kOpBf16Fwd = 4,
          kOpTgmm = 5, kOpDx = 6, kOpFp8Int4 = 7, kNumOps = 8 };

// FP8 forward kernels.
enum Fp8Kernel { kKerAuto = 0, kKerWs = 1, kKerUniform = 2, kKerRowResident = 3 };

// One configuration; 0 in a field means "the library's choice" (an override)
// and is never left in a resolved configuration that uses the field.
struct TileConfig {
    int kernel;     // FP8: Fp8Kernel
    int waves;      // warp-specialised FP8: 8, 12 or 16
    int tile_m;     // FP8 rows per tile: 48 or 64
    int tile_n;     // FP8 columns per workgroup tile: 128, 256 or 512
    int depth;      // warp-specialised FP8: steps of weights in flight (1, 2)
    int residency;  // bf16: workgroups per CU the registers allow (2, 3)
    int placement;  // warp-specialised FP8: 1 consecutive items per XCD, 2 each group's items
                    // on one XCD; tgmm: 1 groups contiguous per XCD, 2 spread over XCDs by
                    // size class; bf16 forward and dX: 1 row tiles aligned to absolute rows,
                    // 2 row tiles starting at each group's first row
};

// The override set for op (all zero when none); set_tile_override(op, NULL)
// clears it.  op must be a valid Op.
TileConfig tile_override(int op);
void set_tile_override(int op, const TileConfig* cfg);

// The configuration a call of op would run (override applied); false, with
// a reason, when the override does not fit this shape.  lhs_kind: 0 E4M3
// codes, 1 bf16, 2 fp32; write_q: the call also writes the LHS codes.
bool resolve_tile_config(int op, int64_t M, int64_t K, int64_t N, int64_t G, int lhs_kind,
                         bool out_bf16, bool write_q, TileConfig* out, const char** why);

}  // namespace gmm
