// Internal declarations shared by the C-ABI layer and the kernel translation unit.
#pragma once
#include <hip/hip_runtime.h>

namespace fa2 {

// Launch shape of one kernel instance.
struct TileShape {
    int rows_per_block;   // query rows per workgroup (BM)
    int keys_per_tile;    // key rows per K/V tile (BN)
    int threads;          // threads per workgroup (64 per wave)
    int lds_bytes;        // dynamic LDS per workgroup
};

// Shape used for head dimension D (64 or 128).
TileShape tile_shape(int D, int causal);

struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, S, D;
    int causal;
    float scale;
};

// Enqueues the kernel for already-validated arguments; returns the launch status.
hipError_t launch_forward(const LaunchArgs& a, hipStream_t stream);

}  // namespace fa2
