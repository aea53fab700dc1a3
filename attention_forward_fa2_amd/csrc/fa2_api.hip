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

bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Limits of the kernel's index arithmetic: row and key indices are 32-bit and
// so is a row index plus a window side (each below 2^29 plus one tile), a
// workgroup id is 31-bit, and a lane's byte offset into one K/V ring stage (up
// to 64 rows of the row stride) is 32-bit. The grid is bounded with the
// smallest workgroup height any shape has, so the limit holds for whichever
// shape the launch picks.
int overflow_status(long long units, int S, long long row_stride_kv, int D) {
    if (S >= (1 << 29)) return FA2_ERR_OVERFLOW;
    const long long rows = fa2::min_rows_per_block(D);
    const long long blocks = units * ((S + rows - 1) / rows);
    if (units > 0x7fffffffll || blocks > 0x7fffffffll) return FA2_ERR_OVERFLOW;
    if (row_stride_kv * 2 * 64 >= (1ll << 32)) return FA2_ERR_OVERFLOW;
    return FA2_OK;
}

int window_dropout_status(int window_left, int window_right, float dropout_p) {
    if (window_left < -1 || window_right < -1) return FA2_ERR_ARG;
    if (!std::isfinite(dropout_p) || dropout_p < 0.0f || !(dropout_p < 1.0f)) return FA2_ERR_ARG;
    return FA2_OK;
}

int heads_status(int H, int H_kv, int D) {
    if (H < 1 || H_kv < 1 || H % H_kv != 0 || (D != 64 && D != 128)) return FA2_ERR_SHAPE;
    return FA2_OK;
}

int scale_status(float scale) {
    return (!std::isfinite(scale) || !(scale > 0.0f)) ? FA2_ERR_SCALE : FA2_OK;
}

// o and lse must not overlap q, k, v (or each other; or the sequence table).
int alias_status(const void* q, size_t nq, const void* k, const void* v, size_t nkv, const void* o,
                 const void* lse, size_t nl, const void* cu, size_t ncu) {
    const void* ins[3] = {q, k, v};
    const size_t nin[3] = {nq, nkv, nkv};
    for (int i = 0; i < 3; ++i)
        if (ranges_overlap(o, nq, ins[i], nin[i]) || ranges_overlap(lse, nl, ins[i], nin[i]))
            return FA2_ERR_ALIAS;
    if (ranges_overlap(o, nq, lse, nl)) return FA2_ERR_ALIAS;
    if (cu && (ranges_overlap(o, nq, cu, ncu) || ranges_overlap(lse, nl, cu, ncu))) return FA2_ERR_ALIAS;
    return FA2_OK;
}

// Every check of the dense entry points that needs no GPU, in the order
// documented in fa2.h.
int validate_dense(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                   int H_kv, int S, int D, int window_left, int window_right, float dropout_p, float scale) {
    if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
    if (B < 1 || S < 1) return FA2_ERR_SHAPE;
    int st = heads_status(H, H_kv, D);
    if (st != FA2_OK) return st;
    if ((st = scale_status(scale)) != FA2_OK) return st;
    if ((st = window_dropout_status(window_left, window_right, dropout_p)) != FA2_OK) return st;
    if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(o) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return FA2_ERR_ALIGN;
    if ((st = overflow_status((long long)B * H, S, D, D)) != FA2_OK) return st;
    const size_t nq = (size_t)B * H * S * D * 2, nkv = (size_t)B * H_kv * S * D * 2, nl = (size_t)B * H * S * 4;
    return alias_status(q, nq, k, v, nkv, o, lse, nl, nullptr, 0);
}

int validate_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const int* cu_seqlens, int num_seqs, int total, int max_seqlen, int H, int H_kv, int D,
                    int window_left, int window_right, float dropout_p, float scale) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA2_ERR_NULLPTR;
    if (num_seqs < 1 || total < 1 || max_seqlen < 1) return FA2_ERR_SHAPE;
    int st = heads_status(H, H_kv, D);
    if (st != FA2_OK) return st;
    if ((st = scale_status(scale)) != FA2_OK) return st;
    if ((st = window_dropout_status(window_left, window_right, dropout_p)) != FA2_OK) return st;
    if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(o) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
        return FA2_ERR_ALIGN;
    if ((st = overflow_status((long long)num_seqs * H, max_seqlen, (long long)H_kv * D, D)) != FA2_OK) return st;
    if ((long long)H * D >= (1ll << 31)) return FA2_ERR_OVERFLOW;
    {
        // the packed grid rounds the (sequence, K/V head) units up to a multiple
        // of 8; bounded with the smallest workgroup height (packed causal
        // batches of short sequences take the half-height shape)
        const long long rows = fa2::min_rows_per_block(D);
        const long long units8 = ((long long)num_seqs * H_kv + 7) / 8 * 8;
        const long long nqt = (max_seqlen + rows - 1) / rows;
        if (units8 * nqt * (H / H_kv) > 0x7fffffffll) return FA2_ERR_OVERFLOW;
    }
    const size_t nq = (size_t)total * H * D * 2, nkv = (size_t)total * H_kv * D * 2, nl = (size_t)total * H * 4;
    return alias_status(q, nq, k, v, nkv, o, lse, nl, cu_seqlens, (size_t)(num_seqs + 1) * 4);
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

int run(const fa2::LaunchArgs& a, void* stream) {
    const int st = check_device();
    if (st != FA2_OK) return st;
    if (fa2::launch_forward(a, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_LAUNCH;
    return FA2_OK;
}

}  // namespace

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
                       int D, int causal, float scale, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
    if (causal != 0 && causal != 1) return FA2_ERR_SHAPE;
    const int st = validate_dense(q, k, v, o, lse, B, H, H, S, D, -1, causal ? 0 : -1, 0.0f, scale);
    if (st != FA2_OK) return st;
    fa2::LaunchArgs a{q, k, v, o, lse, nullptr, B, H, H, S, D, 0, -1, causal ? 0 : -1, scale, 0.0f, 0ull, 0u};
    return run(a, stream);
}

extern "C" int fa2_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                          int S, int D, int window_left, int window_right, float dropout_p,
                          unsigned long long seed, unsigned int offset, float scale, void* stream) {
    const int st = validate_dense(q, k, v, o, lse, B, H, H_kv, S, D, window_left, window_right, dropout_p, scale);
    if (st != FA2_OK) return st;
    fa2::LaunchArgs a{q, k, v, o, lse, nullptr, B, H, H_kv, S, D, 0, window_left, window_right,
                      scale, dropout_p, seed, offset};
    return run(a, stream);
}

extern "C" int fa2_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int num_seqs, int total, int max_seqlen, int H, int H_kv,
                              int D, int window_left, int window_right, float dropout_p, unsigned long long seed,
                              unsigned int offset, float scale, void* stream) {
    const int st = validate_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, total, max_seqlen, H, H_kv, D,
                                   window_left, window_right, dropout_p, scale);
    if (st != FA2_OK) return st;
    fa2::LaunchArgs a{q, k, v, o, lse, cu_seqlens, num_seqs, H, H_kv, max_seqlen, D, total,
                      window_left, window_right, scale, dropout_p, seed, offset};
    return run(a, stream);
}

extern "C" const char* fa2_strerror(int status) {
    switch (status) {
        case FA2_OK: return "ok";
        case FA2_ERR_NULLPTR: return "a tensor pointer is NULL";
        case FA2_ERR_SHAPE:
            return "sizes must be >= 1, D must be 64 or 128, H a multiple of H_kv, causal 0 or 1";
        case FA2_ERR_SCALE: return "scale must be finite and > 0";
        case FA2_ERR_ALIGN:
            return "q, k, v and o must be 16-byte aligned, lse and cu_seqlens 4-byte aligned";
        case FA2_ERR_OVERFLOW:
            return "the sequence length must be < 2^29 and the grid must fit in 2^31-1 workgroups";
        case FA2_ERR_ALIAS: return "o or lse overlaps an input or each other";
        case FA2_ERR_DEVICE: return "there is no current HIP device, or it is not a gfx950 GPU";
        case FA2_ERR_LAUNCH: return "the kernel launch failed";
        case FA2_ERR_ARG: return "window sizes must be >= -1 and the dropout probability in [0, 1)";
        default: return "unknown status";
    }
}

extern "C" int fa2_kernel_config(int B, int H, int S, int D, int causal, int* rows_per_block, int* keys_per_tile,
                                 int* threads_per_block, long long* blocks, int* lds_bytes) {
    if (B < 1 || S < 1 || (causal != 0 && causal != 1)) return FA2_ERR_SHAPE;
    int st = heads_status(H, H, D);
    if (st == FA2_OK) st = overflow_status((long long)B * H, S, D, D);
    if (st != FA2_OK) return st;
    const fa2::TileShape ts = fa2::dense_tile_shape(D, (long long)B * H, S, -1, causal ? 0 : -1);
    if (rows_per_block) *rows_per_block = ts.rows_per_block;
    if (keys_per_tile) *keys_per_tile = ts.keys_per_tile;
    if (threads_per_block) *threads_per_block = ts.threads;
    if (blocks) *blocks = (long long)B * H * ((S + ts.rows_per_block - 1) / ts.rows_per_block);
    if (lds_bytes) *lds_bytes = ts.lds_bytes;
    return FA2_OK;
}
