// Internal declarations shared by the C-ABI layer and the kernel translation unit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

// Launch shape of one kernel instance.
struct TileShape {
    int rows_per_block;   // query rows per workgroup (BM)
    int keys_per_tile;    // key rows per LDS ring stage
    int threads;          // threads per workgroup (64 per wave)
    int lds_bytes;        // dynamic LDS per workgroup
};

// The full-height shape for head dimension D (64 or 128).
TileShape tile_shape(int D);

// The fewest query rows per workgroup of any shape a launch at head dimension
// D may pick (the half-height shapes). Grid-size limits are checked with it, so
// they hold whichever shape the launch selects.
int min_rows_per_block(int D);

// The shape a dense launch of `units` (batch*head) heads of length S uses.
TileShape dense_tile_shape(int D, long long units, int S, int window_left, int window_right);

// Already-validated arguments of one forward pass.
struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int* cu_seqlens;   // device [B+1] start rows of packed sequences, or null (dense)
    int B;                   // batch (dense) or number of packed sequences
    int H, H_kv, S, D;       // S: sequence length (dense) or longest sequence (packed)
    int total;               // rows of the packed tensors (packed only)
    int window_left;         // < 0: unbounded
    int window_right;        // < 0: unbounded; (-1, 0) is causal
    float scale;
    float dropout_p;         // 0 <= p < 1; 0 disables dropout
    unsigned long long seed;
    unsigned int offset;
};

// Keep threshold of a dropout probability: a key is kept when its 16-bit draw
// is >= floor(p * 2^16) (clamped to 2^16 - 1).
uint32_t drop_threshold(float p);

// Enqueues the kernel for already-validated arguments; returns the launch status.
hipError_t launch_forward(const LaunchArgs& a, hipStream_t stream);

}  // namespace fa2
