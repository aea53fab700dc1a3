// Index arithmetic of the forward kernel that involves no wave-level
// operation, for host and device: the kernel's argument block, the workgroup ->
// (head, query tile) mapping, the LDS swizzles, and the per-lane offsets of the
// K/V loads and of the LDS reads. The kernel includes this header, and so does a
// host-only probe library (tests/index_probe), through which the CPU tests
// check their emulation of these formulas against this code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {
namespace {

// Everything the kernel needs about one launch. Tensors are addressed through
// element strides so that one kernel serves the dense [B,H,S,D] layout and the
// packed variable-length layout [total,H,D]:
//   element (b, h, row, d) of q/o at  q + b*q_sb + h*q_sh + (start_b + row)*q_sr + d
//   element (b, hk, row, d) of k/v at k + b*kv_sb + hk*kv_sh + (start_b + row)*kv_sr + d
//   lse (b, h, row)                at  lse + b*l_sb + h*l_sh + start_b + row
// where start_b = cu[b] and the sequence length len_b = cu[b+1] - cu[b] when a
// sequence table cu is given, and start_b = 0, len_b = S otherwise.
struct KernelArgs {
    const _Float16* q;
    const _Float16* k;
    const _Float16* v;
    _Float16* o;
    float* lse;
    const int* cu;        // [nseq+1] start rows of packed sequences, or null
    long long q_sb, q_sh, kv_sb, kv_sh, l_sb, l_sh;
    int q_sr, kv_sr;
    int S;                // sequence length (dense) or longest sequence (packed)
    int total;            // rows of the packed tensors (packed only)
    int H;                // query heads
    int group;            // query heads per K/V head (H / H_kv)
    int BH;               // sequences * H
    int BHkv;             // sequences * H_kv
    int nqt;              // query tiles per (sequence, head)
    int nblocks;          // BH * nqt
    int wl, wr;           // local window: keys i-wl .. i+wr (window kernels only)
    float c;              // scale * log2(e)
    float out_scale;      // 1/(1-p) with dropout, else 1
    uint32_t drop_thr;    // a key is kept when its 16-bit draw is >= drop_thr
    uint32_t seed_lo, seed_hi, offset;
    int serp;             // one-round causal grids: workgroups per serpentine band (CUs per XCD), else 0
    int lpt;              // packed launches: walk the sequences longest first (at most 64 sequences)
};

enum MaskKind { kNoMask = 0, kCausal = 1, kWindow = 2 };

// XOR swizzles of the 16-byte chunk index within a row, chosen so that the 16
// rows read by one ds_read_b128 quarter-wave (K) and the 8 rows x 2 chunks read
// by one ds_read_b64_tr_b16 half-wave (V) land on distinct 16-byte bank groups
// of a 256-byte bank window.
template <int D>
__host__ __device__ __forceinline__ int swz_k(int row) {
    return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
template <int D>
__host__ __device__ __forceinline__ int swz_v(int row) {
    return D == 64 ? (((row >> 1) & 3) << 1) : ((row & 7) << 1);
}
// V swizzle of the 32x32x16 path (D = 64): one transposing-read half-wave
// reads 4 consecutive rows x 4 consecutive chunks (64 bytes of each row); rows
// of equal parity share a 256-byte bank window, so rows 2 and 3 of each group
// of 4 take the other half of the row: chunk index xor 4.
__host__ __device__ __forceinline__ int swz_v32(int row) { return ((row >> 1) & 1) << 2; }

// Per-lane source offsets (bytes, within a stage) of a lane's direct-to-LDS
// loads: load i fills LDS chunk c = (i*NW + wave)*64 + lane, i.e. stage row
// r = c / CPR and physical chunk pc = c % CPR (CPR = D/8 chunks of 16 bytes per
// row), from the logical chunk pc ^ swz(r) of key row k0 + r. Successive loads
// of a lane are NW*64/CPR rows apart, a multiple of the 16-row swizzle period,
// so one lane offset per tensor serves all of them. row0 is the lane's first
// stage row; kv_sr the K/V row stride in elements.
template <int D, int NW, bool MF32>
__host__ __device__ __forceinline__ void lane_load_offsets(int wave, int lane, int kv_sr, int& row0,
                                                           uint32_t& offK, uint32_t& offV) {
    constexpr int CPR = D / 8;
    static_assert((NW * 64 / CPR) % 16 == 0, "loads of a lane must keep the swizzle phase");
    row0 = (wave * 64 + lane) / CPR;
    const int pc0 = lane % CPR;
    offK = 2u * (row0 * kv_sr + 8 * (pc0 ^ swz_k<D>(row0)));
    offV = 2u * (row0 * kv_sr + 8 * (pc0 ^ (MF32 ? swz_v32(row0) : swz_v<D>(row0))));
}

// LDS read offsets (bytes) of the 16x16x32 path that do not depend on the tile:
// the K swizzle of rows 16*kb + l16 depends on l16 only, the V swizzle of rows
// 32*kc + 4g + l16/4 (+16) on g and l16 only (l16 = lane%16, g = lane/16). The
// k-step kk (K) and the column block db (V) only flip the address bits the
// swizzle acts on, which the row and lane terms leave clear, so
//   offset(K, kk) = rdK0 ^ (kk << 6),   offset(V, db) = rdV0 ^ (db << 5):
// one register per tensor instead of one per k-step or column block.
template <int D>
__host__ __device__ __forceinline__ void lds_read_bases(int lane, uint32_t& rdK0, uint32_t& rdV0) {
    const int l16 = lane & 15, g = lane >> 4;
    rdK0 = 2u * (l16 * D + 8 * (g ^ swz_k<D>(l16)));
    const int r0 = 4 * g + (l16 >> 2);
    rdV0 = 2u * (r0 * D + 8 * (((l16 & 3) >> 1) ^ swz_v<D>(r0)) + 4 * (l16 & 1));
}

// Workgroup -> (sequence*H + head, query tile). Consecutive workgroup ids are
// dispatched round-robin to the 8 XCDs, each with its own L2, so the mapping
// keeps the workgroups that read one K/V head on one XCD:
//  * non-causal and windowed: XCD x gets a contiguous run of (head, tile) pairs
//    in head-major order, i.e. all query tiles of a few heads; heads that share
//    a K/V head are adjacent;
//  * causal with (sequences * K/V heads) a multiple of 8: XCD x gets K/V heads
//    x, x+8, ... with all query heads of each, and walks them heaviest query
//    tile first (the last tiles see the most keys), so the long workgroups
//    start early and each K/V head has several tiles in flight on one XCD.
//    When the whole grid is resident at once (one round, nothing refills a
//    compute unit), the walk is a serpentine instead: bands of a.serp
//    consecutive workgroups of an XCD (one per compute unit of the XCD) run
//    alternately heaviest-first and lightest-first, so that the workgroups a
//    compute unit receives, one from each band, add up to the same number of
//    keys on every compute unit;
//  * causal otherwise: heaviest tiles first over all heads;
//  * packed sequences of different lengths: (sequence, K/V head) unit u goes
//    to XCD u mod 8, so that with 8 or more heads every XCD gets its share of
//    every sequence whatever the lengths; an XCD walks its units one by one
//    (all query tiles of a unit and all query heads of its group together;
//    causal: heaviest tile first). With at most 64 sequences the units are
//    numbered longest sequence first (each workgroup ranks the lengths from
//    the table itself), so that the long workgroups start early and short
//    ones fill the end of the launch. The grid then has
//    ceil(units/8)*8*nqt*group workgroups, and those past the last unit, or
//    past the end of a short sequence, exit at once. Returns false for a
//    workgroup with no work. rank_of(nseq, rho) names the sequence that ranks
//    rho-th by length, longest first (ties by index), among the first nseq
//    sequences of the table; it is called only for packed launches with lpt set.
template <int MASK, class RankOf>
__host__ __device__ __forceinline__ bool map_block(const KernelArgs& a, int bid, int& bh, int& qt, RankOf rank_of) {
    const int xcd = bid & 7, slot = bid >> 3;
    if (a.cu) {
        const int per_unit = a.nqt * a.group;
        int kvu = xcd + 8 * (slot / per_unit);
        const int rem = slot % per_unit;
        if (kvu >= a.BHkv) return false;
        if (a.lpt) {
            const int H_kv = a.H / a.group;
            kvu = rank_of(a.BHkv / H_kv, kvu / H_kv) * H_kv + kvu % H_kv;
        }
        qt = rem / a.group;
        if (MASK == kCausal) qt = a.nqt - 1 - qt;
        bh = kvu * a.group + rem % a.group;
        return true;
    }
    if (MASK == kCausal && (a.BHkv & 7) == 0) {
        const int per_tile = (a.BHkv >> 3) * a.group;  // query heads per XCD
        int s = slot;
        if (a.serp) {
            const int band = s / a.serp;  // complete odd bands run backwards
            if ((band & 1) && (band + 1) * a.serp <= (a.nblocks >> 3)) s = band * a.serp + (a.serp - 1 - s % a.serp);
        }
        qt = a.nqt - 1 - s / per_tile;
        const int r = s % per_tile;
        bh = (xcd + 8 * (r / a.group)) * a.group + r % a.group;
        return true;
    }
    const int per = a.nblocks >> 3, rem = a.nblocks & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    if (MASK == kCausal) {
        qt = a.nqt - 1 - logical / a.BH;
        bh = logical % a.BH;
    } else {
        bh = logical / a.nqt;
        qt = logical % a.nqt;
    }
    return true;
}

}  // namespace
}  // namespace fa2
