// MFMA tier dispatcher: tile table and routing of each op to its kernel
// instantiations (mfma_fwd.hip, mfma_dx.hip, mfma_dw.hip, mfma_grouped.hip;
// the kernel itself is in mfma_kernel.hpp).
#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

hipError_t launch_mfma_fwd(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid,
                           hipStream_t s);
hipError_t launch_mfma_dx(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid,
                          hipStream_t s);
hipError_t launch_mfma_dw(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid,
                          hipStream_t s);
hipError_t launch_mfma_grouped(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid,
                               hipStream_t s);

const TileShape *mfma_tile(int id) {
    static const TileShape shapes[] = {
        {1, 256, 256}, {2, 256, 192}, {3, 256, 128}, {4, 128, 128}, {5, 128, 96},
        {6, 64, 64},   {7, 128, 256}, {9, 128, 192}, {10, 256, 96},
        // eight-wave workgroups
        {11, 256, 192}, {12, 256, 256}, {13, 256, 128}, {14, 128, 256}, {15, 128, 128},
    };
    // ids 40 + i: the direct-load kernel on base tile i (same shape)
    static const TileShape dl[] = {
        {41, 256, 256}, {42, 256, 192}, {43, 256, 128}, {44, 128, 128}, {45, 128, 96},
        {46, 64, 64},   {47, 128, 256}, {49, 128, 192}, {50, 256, 96},  {51, 256, 192},
        {52, 256, 256}, {53, 256, 128}, {54, 128, 256}, {55, 128, 128},
        {48, 96, 96},   {56, 192, 256}, {57, 96, 96},  {120, 64, 32}, {121, 32, 32},
    };
    // ids 100 + i: the direct-load kernel with copies spread between MFMAs
    static const TileShape dls[] = {
        {104, 128, 128}, {105, 128, 96}, {108, 96, 96}, {111, 256, 192}, {112, 256, 256},
        {114, 128, 256}, {115, 128, 128}, {116, 192, 256},
    };
    // ids 200 + i / 300 + i: the direct-load kernel with double- / quadruple-depth stages
    static const TileShape dld[] = {{220, 64, 32}, {321, 32, 32}};
    for (const TileShape &s : dld)
        if (s.id == id) return &s;
    for (const TileShape &s : dls)
        if (s.id == id) return &s;
    for (const TileShape &s : shapes)
        if (s.id == id) return &s;
    for (const TileShape &s : dl)
        if (s.id == id) return &s;
    return nullptr;
}

hipError_t launch_mfma_gemm(const MfmaArgs &p, int tile_id, int dt, int layout, int epi,
                            hipStream_t s) {
    const bool seg = p.offsets != nullptr, red = p.red_offsets != nullptr;
    int64_t grid;
    if (seg) grid = seg_grid_rows(p.seg_tiles) * p.tiles_j;
    else if (red) grid = p.n_experts * p.tiles_i * p.tiles_j;
    else grid = p.tiles_i * p.tiles_j * p.nchunks;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (seg && layout == 3 && epi == 0) return launch_mfma_grouped(p, tile_id, dt, 0, grid, s);
    if (seg && layout == 1 && epi == 0) return launch_mfma_grouped(p, tile_id, dt, 1, grid, s);
    if (red && layout == 0 && epi == 2) return launch_mfma_grouped(p, tile_id, dt, 2, grid, s);
    if (seg || red) return hipErrorInvalidValue;
    if (layout == 1 && epi == 0) return launch_mfma_fwd(p, tile_id, dt, epi, grid, s);
    if (layout == 3 && epi == 0) return launch_mfma_dx(p, tile_id, dt, epi, grid, s);
    if (layout == 0 && (epi == 0 || epi == 1)) return launch_mfma_dw(p, tile_id, dt, epi, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bi
