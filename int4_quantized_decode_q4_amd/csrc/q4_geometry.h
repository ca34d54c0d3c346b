// q4_geometry.h -- geometry of the device layout (version 1), shared by the
// host API and the kernels of libq4.  The rule is stated in include/q4.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace q4 {

struct Geometry {
    int L;              // lanes of a wavefront that share one row
    int CG;             // groups of 32 codes per lane per row, per pass
    int P;              // passes over k
    int TR;             // rows per tile = 2 * 64 / L
    int64_t tiles;      // ceil(rows / TR)
    int64_t pass_bytes; // CG * 2304 (int3: CG * 1792)
    int64_t tile_bytes; // P * pass_bytes
};

// Returns false for an invalid shape.  Choice of (L, CG): least L*CG that
// covers the groups of one pass, ties to the larger L (more lanes along k,
// fewer rows per wavefront instruction).
__host__ __device__ inline bool layout_geometry(int64_t rows, int64_t k, Geometry *g)
{
    if (rows < 1 || k < 32 || (k % 32) != 0)
        return false;
    const int64_t groups = k / 32;
    const int64_t passes = (groups + 255) / 256;
    const int64_t per_pass = (groups + passes - 1) / passes;
    int best_l = 0, best_cg = 0;
    int64_t best_cover = 0;
    for (int l = 64; l >= 1; l >>= 1)
        for (int cg = 1; cg <= 4; ++cg) {
            const int64_t cover = (int64_t)l * cg;
            if (cover >= per_pass && (best_l == 0 || cover < best_cover)) {
                best_l = l;
                best_cg = cg;
                best_cover = cover;
            }
        }
    g->L = best_l;
    g->CG = best_cg;
    g->P = (int)passes;
    g->TR = 2 * (64 / best_l);
    g->tiles = (rows + g->TR - 1) / g->TR;
    g->pass_bytes = (int64_t)best_cg * 2304;
    g->tile_bytes = passes * g->pass_bytes;
    return true;
}

// The int3 layout: the same tiles and lane mapping, with 12-byte lane units
// (3 words of codes per group instead of 4), so a pass is CG * 1792 bytes.
__host__ __device__ inline bool layout_geometry3(int64_t rows, int64_t k, Geometry *g)
{
    if (!layout_geometry(rows, k, g))
        return false;
    g->pass_bytes = (int64_t)g->CG * 1792;
    g->tile_bytes = g->P * g->pass_bytes;
    return true;
}

}  // namespace q4
