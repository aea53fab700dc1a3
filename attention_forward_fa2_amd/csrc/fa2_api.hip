// C ABI of the FlashAttention-2 forward library: argument validation, the
// gfx950 device check and kernel dispatch. Declared in include/fa2.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/fa2.h"
#include "fa2_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = other
std::atomic<int> g_device_kind[kMaxDevices];

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int shape_status(int B, int H, int S, int D, int causal) {
    if (B < 1 || H < 1 || S < 1 || (D != 64 && D != 128) || (causal != 0 && causal != 1))
        return FA2_ERR_SHAPE;
    return FA2_OK;
}

int overflow_status(int B, int H, int S, int D, int causal) {
    if ((long long)S * D >= (1ll << 31)) return FA2_ERR_OVERFLOW;
    const fa2::TileShape ts = fa2::tile_shape(D, causal);
    const long long blocks = (long long)B * H * ((S + ts.rows_per_block - 1) / ts.rows_per_block);
    if (blocks > 0x7fffffffll) return FA2_ERR_OVERFLOW;
    return FA2_OK;
}

// Every check that needs no GPU, in the order documented in fa2.h.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
             int S, int D, int causal, float scale) {
    if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
    int st = shape_status(B, H, S, D, causal);
    if (st != FA2_OK) return st;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA2_ERR_SCALE;
    const uintptr_t mis = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o)) & 15u;
    if (mis || (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA2_ERR_ALIGN;
    st = overflow_status(B, H, S, D, causal);
    if (st != FA2_OK) return st;
    const size_t tensor_bytes = (size_t)B * H * S * D * 2;
    const size_t lse_bytes = (size_t)B * H * S * 4;
    if (ranges_overlap(o, tensor_bytes, q, tensor_bytes) || ranges_overlap(o, tensor_bytes, k, tensor_bytes) ||
        ranges_overlap(o, tensor_bytes, v, tensor_bytes) || ranges_overlap(lse, lse_bytes, q, tensor_bytes) ||
        ranges_overlap(lse, lse_bytes, k, tensor_bytes) || ranges_overlap(lse, lse_bytes, v, tensor_bytes) ||
        ranges_overlap(o, tensor_bytes, lse, lse_bytes))
        return FA2_ERR_ALIAS;
    return FA2_OK;
}

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int kind = g_device_kind[dev].load(std::memory_order_relaxed);
        if (kind == 1) return FA2_OK;
        if (kind == 2) return FA2_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA2_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_device_kind[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? FA2_OK : FA2_ERR_DEVICE;
}

}  // namespace

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
                       int D, int causal, float scale, void* stream) {
    int st = validate(q, k, v, o, lse, B, H, S, D, causal, scale);
    if (st != FA2_OK) return st;
    st = check_device();
    if (st != FA2_OK) return st;
    fa2::LaunchArgs a{q, k, v, o, lse, B, H, S, D, causal, scale};
    if (fa2::launch_forward(a, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_LAUNCH;
    return FA2_OK;
}

extern "C" const char* fa2_strerror(int status) {
    switch (status) {
        case FA2_OK: return "ok";
        case FA2_ERR_NULLPTR: return "a tensor pointer is NULL";
        case FA2_ERR_SHAPE: return "B, H and S must be >= 1, D must be 64 or 128, causal must be 0 or 1";
        case FA2_ERR_SCALE: return "scale must be finite and > 0";
        case FA2_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned and lse 4-byte aligned";
        case FA2_ERR_OVERFLOW: return "S*D must be < 2^31 and the grid must fit in 2^31-1 workgroups";
        case FA2_ERR_ALIAS: return "o or lse overlaps an input or each other";
        case FA2_ERR_DEVICE: return "the current HIP device is not a gfx950 GPU";
        case FA2_ERR_LAUNCH: return "the kernel launch failed";
        default: return "unknown status";
    }
}

extern "C" int fa2_kernel_config(int B, int H, int S, int D, int causal, int* rows_per_block, int* keys_per_tile,
                                 int* threads_per_block, long long* blocks, int* lds_bytes) {
    int st = shape_status(B, H, S, D, causal);
    if (st == FA2_OK) st = overflow_status(B, H, S, D, causal);
    if (st != FA2_OK) return st;
    const fa2::TileShape ts = fa2::tile_shape(D, causal);
    if (rows_per_block) *rows_per_block = ts.rows_per_block;
    if (keys_per_tile) *keys_per_tile = ts.keys_per_tile;
    if (threads_per_block) *threads_per_block = ts.threads;
    if (blocks) *blocks = (long long)B * H * ((S + ts.rows_per_block - 1) / ts.rows_per_block);
    if (lds_bytes) *lds_bytes = ts.lds_bytes;
    return FA2_OK;
}
