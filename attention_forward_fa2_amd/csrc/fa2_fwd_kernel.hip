// FlashAttention-2 forward for gfx950 (MI355X, CDNA4).
//
// Method: the page "CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy 与
// TiledMMA" (cited as [CuTe-FA2]). Each workgroup owns a block of query rows
// and scans K/V in tiles, keeping per query row a running max m, a running sum l
// and an unnormalised output o (§"教学配置：一块 CTA 做什么"), updated per tile by
// the equations of §"沿 C fragment 做 Online Softmax"; O = o / l at the end.
// Every wave owns its query rows from the scores to the output, so waves never
// combine partial results (the Q split of §"TiledMMA：把四个 warp 只铺在 M 维").
//
// gfx950 mapping (lane layouts measured on the device with a probe that sends
// integer matrices through the instructions and compares with a CPU product):
//   * MFMA v_mfma_f32_16x16x32_f16. For a 16x32 A, 32x16 B and 16x16 C:
//       A[i][k] -> lane i + 16*(k/8), element k%8
//       B[k][j] -> lane j + 16*(k/8), element k%8
//       C[i][j] -> lane j + 16*(i/4), element i%4
//   * Scores are computed transposed, S^T = K Q^T (A = K tile from LDS, B = Q^T
//     held in registers for the whole scan). A lane then holds one query column
//     (lane%16) and keys 4*(lane/16)+0..3 of every 16-key block.
//   * Output is accumulated transposed, O^T += V^T P^T. The B operand P^T needs,
//     per lane, one query (lane%16) and 8 keys of a 32-key chunk; taking keys
//     {4g..4g+3} from the first 16-key block and {16+4g..16+4g+3} from the
//     second (g = lane/16) makes the S^T accumulator registers, converted to
//     fp16, exactly that operand: no lane exchange and no LDS round trip
//     (the counterpart of the C-to-A reinterpretation in §"全文最关键的一步").
//     The A operand V^T uses the same key order; it is read from the row-major
//     V tile with the transposing LDS read ds_read_b64_tr_b16, which gives lane i
//     of a 16-lane group 4 consecutive rows of column i (§"V 的转置只发生在视图里":
//     V is never transposed in memory).
//   * The row max combines the 4 lanes that share a query (lanes l, l^16,
//     l^32, l^48) with v_permlane16_swap / v_permlane32_swap: the reduction
//     group follows the accumulator ownership (§"把 lane 公式真正写出来"). The
//     row sum is either kept per lane (v_dot2 on the fp16 P) and combined the
//     same way at the end, or taken on the matrix unit by an MFMA with an
//     all-ones A operand, which hands every lane its query's full sum.
//   * K and V tiles go HBM -> LDS with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4, LDS destination = base + 16*lane) into a
//     two-stage ring (§"多 Stage 流水"); the tile for step t+1 is in flight while
//     step t computes. The XOR swizzle of 16-byte chunks is applied on the
//     source side because the LDS side of these loads is lane-linear.
//   * Softmax runs in base 2: the max is taken on raw scores, then
//     p = 2^(s*c - m*c) with c = scale*log2(e), one FMA and one v_exp_f32 per
//     score (§"沿 C fragment 做 Online Softmax", closing paragraph).
//
// The same kernel serves the features §"哪些结论可以迁移，哪些只是本例特例" lists
// for a production FA2: query heads sharing K/V heads (GQA/MQA: the K/V head
// index in the base address), local windows (a mask kind that bounds the ring
// stages a workgroup loads and the tiles each wave computes), packed sequences
// of different lengths (tensors addressed through strides, sequence start and
// length read from a table), and dropout on P (a counter-based generator,
// Philox4x32-10, evaluated in registers).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <type_traits>

#include "fa2_index.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr double kLog2e = 1.44269504088896340736;
// Finite start value of the running reference (base-2 units, i.e. a score times
// c): exp2(m0 - m*c) is exactly 0 for any real score m, and a row whose keys
// were all masked so far keeps alpha = 1, p = 0.
constexpr float kMaxInit = -1.0e30f;
// A row sum of fp16 probabilities (a lane's partial sum, or the tile's full
// sum) below this bound means none of them overflowed fp16 (largest finite
// 65504).
constexpr float kSpeculateLimit = 32768.0f;
// A rebase sets the reference this far (base-2 units) above the tile's row
// maximum: the tile's probabilities are then at most 2^-8, which keeps every
// key within 6 units of the maximum in the normal fp16 range, and later tiles
// may rise 15 + 8 units above that maximum before a p could overflow, which
// halves the rebases of peaked rows (scores with a standard deviation of 13
// base-2 units: 4.4 -> 2.0 per 32-row wave over 1000 keys in the fp64 model
// of this rule, with the same error).
#ifndef FA2_REF_HEADROOM
#define FA2_REF_HEADROOM 8.0f
#endif
constexpr float kRefHeadroom = FA2_REF_HEADROOM;

template <int D_, int QB_, int NW_, int BN_, int SUB_, int MF_ = 16>
struct Shape {
    static constexpr int D = D_;
    static constexpr int MF = MF_;            // MFMA shape: 16 (16x16x32) or 32 (32x32x16)
    static constexpr int QB = QB_;            // 16-query blocks per wave
    static constexpr int NW = NW_;            // waves per workgroup
    static constexpr int BN = BN_;            // keys per compute tile
    static constexpr int SUB = SUB_;          // compute tiles per LDS ring stage
    static constexpr int KB = SUB * BN;       // keys per ring stage (one barrier each)
    static constexpr int QW = 16 * QB;        // query rows per wave
    static constexpr int BM = NW * QW;        // query rows per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int NKB = BN / 16;       // 16-key blocks per tile
    static constexpr int NKC = BN / 32;       // 32-key chunks per tile
    static constexpr int DK = D / 32;         // k-steps of one score MFMA block
    static constexpr int DB = D / 16;         // 16-wide column blocks of the output
    static constexpr int CPR = D / 8;         // 16-byte chunks per row
    static constexpr int TILE = BN * D;       // halves per K or V compute tile
    static constexpr int LTILE = SUB * TILE;  // halves per K or V ring stage
    static constexpr int LOADS = LTILE / 8 / 64 / NW;  // 16-byte loads per lane per tensor per stage
    static constexpr int LDS_BYTES = 2 /*stages*/ * 2 /*K,V*/ * LTILE * 2;
    // Occupancy the register allocation targets (waves per SIMD).
    static constexpr int WAVES_PER_SIMD = (D == 64 && QB <= 2) ? 4 : (QB <= 2 ? 2 : 1);
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert((LTILE / 8) % (64 * NW) == 0, "loads must divide evenly among lanes");
    static_assert(BN % 16 == 0, "swizzles repeat every 16 rows, so sub-tiles share them");
    static_assert(MF == 16 || (MF == 32 && D == 64 && QB == 2), "the 32x32x16 path tiles 32 query rows at D = 64");
};


// max / sum over lanes {l, l^16} and {l, l^32}. Both swap results hold the two
// partners in the same order on every lane, so all four lanes of a query get
// bit-identical values.
__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct-to-LDS 16-byte loads. Lane i's 16 bytes land at LDS byte address
// lds_base + 16*i (lds_base must be wave-uniform). Written as inline asm so the
// compiler does not track them: its own tracking of these loads would make every
// later LDS read of the other ring stage wait for them, which removes the
// overlap of the next tile's load with this tile's math. The kernel waits for
// them itself (vmcnt(0)) before the barrier that publishes a stage. M0 carries
// the LDS base; it is an input operand of the asm ("{m0}"), so the compiler sets
// it and knows its value wherever else M0 may be needed.
//   dma_16B_s: address = 64-bit wave-uniform base (SGPRs) + 32-bit lane offset.
//   dma_16B_v: full 64-bit per-lane address.
// Hazards the compiler cannot see through the asm, so the asm pays them itself:
//   * a VALU write of an SGPR (the v_readfirstlane that moves the base into
//     SGPRs) followed by a vector-memory instruction that reads that SGPR
//     needs 5 wait states: s_nop 4 before the SGPR-based load, whatever the
//     compiler scheduled just before the asm;
//   * a write of M0 followed by an LDS-DMA load needs 1 wait state: covered by
//     the same s_nop 4, and by s_nop 0 in the VGPR-addressed form.
__device__ __forceinline__ void dma_16B_s(const void* sbase_in, uint32_t voff, uint32_t lds_base) {
    // The base is wave-uniform; say so, so it is kept in SGPRs as the
    // instruction requires.
    // (readfirstlane returns a signed int: go through uint32_t so the low half
    // is zero-extended, not sign-extended, when it is widened.)
    const uint64_t b = reinterpret_cast<uint64_t>(sbase_in);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const void* sbase = reinterpret_cast<const void*>((hi << 32) | lo);
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "{m0}"(lds_base)
        : "memory");
}
__device__ __forceinline__ void dma_16B_v(const void* src, uint32_t lds_base) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(src), "{m0}"(lds_base)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_void*)p;
}

template <int V>
using Int = std::integral_constant<int, V>;


// Index of the sequence that ranks rho-th by length, longest first (ties by
// index), among nseq <= 64 sequences of a packed table: lane j takes sequence
// j's clamped length, counts the sequences that rank before it, and the lane
// whose count is rho names the sequence. Every wave computes the same answer.
__device__ __forceinline__ int sequence_of_rank(const KernelArgs& a, int nseq, int rho) {
    const int lane = threadIdx.x & 63;
    int len = -1;
    if (lane < nseq) {
        const int s0 = min(max(a.cu[lane], 0), a.total);
        const int s1 = min(max(a.cu[lane + 1], s0), a.total);
        len = min(s1 - s0, a.S);
    }
    int rank = 0;
    for (int i = 0; i < nseq; ++i) {
        const int li = __builtin_amdgcn_readlane(len, i);
        rank += (li > len) || (li == len && i < lane);
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < nseq && rank == rho);
    return hit ? __builtin_ctzll(hit) : 0;
}


// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64-bit products and xors
// on a 4-word counter under a 2-word key that advances by the Weyl constants
// between rounds. Returns the four output words.
struct U32x4 {
    uint32_t w[4];
};
__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input xor in one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return U32x4{{c0, c1, c2, c3}};
}

// Raise the wave priority around the MFMA blocks so the arbiter keeps the matrix
// unit fed from whichever wave has MFMAs ready (a scheduling hint only).
#ifndef FA2_SETPRIO
#define FA2_SETPRIO 1
#endif
// Wave priorities (0..3) for the score MFMAs, the softmax that follows them and
// the PV MFMAs; the priority returns to 0 after the PV block. (2, 1, 1)
// measured best over the workloads, within 2 % of the neighbouring settings.
#ifndef FA2_PRIO_QK
#define FA2_PRIO_QK 2
#endif
#ifndef FA2_PRIO_SM
#define FA2_PRIO_SM 1
#endif
#ifndef FA2_PRIO_PV
#define FA2_PRIO_PV 1
#endif
// 16-key blocks whose score MFMAs are interleaved (1, 2 or 4; see compute_tile).
#ifndef FA2_QK_GROUP
#define FA2_QK_GROUP 4
#endif
// Row sums of P on the matrix unit (an MFMA against an all-ones operand)
// instead of v_dot2 on the VALU: 0 never, 1 always, 2 for D=128 and for
// unmasked D=64 (where it measured faster; elsewhere it was even or slower).
#ifndef FA2_MFMA_ROWSUM
#define FA2_MFMA_ROWSUM 2
#endif

// Debug build (FA2_POISON_LDS=1, a separate library): before each ring stage
// is refilled, every lane overwrites the LDS chunks its own direct-to-LDS loads
// are about to fill with NaN (all bits set) and waits for those writes. A read
// that the wait/barrier protocol fails to order after the loads, or after the
// last reads of the stage's previous tile, then sees NaN, which reaches the
// output. With a correct protocol the outputs are those of the normal build.
#ifndef FA2_POISON_LDS
#define FA2_POISON_LDS 0
#endif

// Occupancy target of the dropout instances at D=64 (waves per SIMD). At 4
// they fit the 128-register budget without spills; 3 (141 registers) was
// measured 11-12 % slower.
#ifndef FA2_DROP_WAVES
#define FA2_DROP_WAVES 4
#endif

template <class SH, int MASK, bool DROP>
__global__ __launch_bounds__(SH::THREADS)
__attribute__((amdgpu_waves_per_eu((DROP && SH::D == 64) ? FA2_DROP_WAVES : SH::WAVES_PER_SIMD)))
void fa2_fwd_kernel(KernelArgs a) {
    constexpr int D = SH::D, QB = SH::QB, NW = SH::NW, BN = SH::BN, QW = SH::QW, BM = SH::BM;
    constexpr int NKB = SH::NKB, NKC = SH::NKC, DK = SH::DK, DB = SH::DB, CPR = SH::CPR;
    constexpr int TILE = SH::TILE, LTILE = SH::LTILE, LOADS = SH::LOADS, SUB = SH::SUB, KB = SH::KB;
    constexpr bool ROWSUM_MFMA = FA2_MFMA_ROWSUM == 1 || (FA2_MFMA_ROWSUM == 2 && (D == 128 || MASK == kNoMask));
    // 32x32x16 MFMAs (D = 64; the dropout instances keep the 16x16x32 path,
    // whose lane pairs share the generator's draws)
    constexpr bool MF32 = SH::MF == 32 && !DROP;

    // LDS ring: [stage][K | V][LTILE] halves; a stage holds SUB compute tiles.
    extern __shared__ __attribute__((aligned(16))) _Float16 smem[];
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int bid = blockIdx.x + blockIdx.y * gridDim.x;  // grid is (x, y) only when x alone is too small
    if (bid >= a.nblocks) return;
    int bh, qt;
    if (!map_block<MASK>(a, bid, bh, qt, [&](int nseq, int rho) { return sequence_of_rank(a, nseq, rho); })) return;
    const int b = bh / a.H, h = bh - b * a.H, hk = h / a.group;

    // This sequence's first row and length. A packed table is read with scalar
    // loads and clamped to the tensors, so a malformed table cannot make the
    // kernel address memory outside them.
    int start = 0, len = a.S;
    if (a.cu) {
        const int s0 = min(max(a.cu[b], 0), a.total);
        const int s1 = min(max(a.cu[b + 1], s0), a.total);
        start = s0;
        len = min(s1 - s0, a.S);
    }
    const int q0 = qt * BM;
    if (q0 >= len) return;  // whole workgroup: no barrier has been reached
    const int qw0 = q0 + wave * QW;
    const int q_sr = a.q_sr, kv_sr = a.kv_sr;

    const _Float16* __restrict__ Qh = a.q + b * a.q_sb + h * a.q_sh + (long long)start * q_sr;
    const _Float16* __restrict__ Kh = a.k + b * a.kv_sb + hk * a.kv_sh + (long long)start * kv_sr;
    const _Float16* __restrict__ Vh = a.v + b * a.kv_sb + hk * a.kv_sh + (long long)start * kv_sr;

    // Keys this workgroup may need, [kbeg, kend), and the ring stages (KB keys
    // each) that hold them.
    const int q_last = min(q0 + BM, len) - 1;
    int kbeg = 0, kend = len;
    if (MASK == kCausal) kend = q_last + 1;
    if (MASK == kWindow) {
        kbeg = max(0, q0 - a.wl);
        kend = min(len, q_last + a.wr + 1);
    }
    const int t_begin = kbeg / KB;
    const int t_end = (kend + KB - 1) / KB;

    // Per-lane source offsets (bytes, within a stage) of this lane's
    // direct-to-LDS loads (lane_load_offsets): one lane offset per tensor serves
    // all LOADS loads of a stage, ROWS_PER_LOAD rows apart; the rest is a scalar
    // step.
    constexpr int ROWS_PER_LOAD = NW * 64 / CPR;
    int row0;
    uint32_t offK, offV;
    lane_load_offsets<D, NW, MF32>(wave, lane, kv_sr, row0, offK, offV);

    // Issue the direct-to-LDS loads of K/V stage t (keys t*KB ..) into ring stage
    // ST. Rows past the end of the sequence (only in the last stage) are clamped
    // to row len-1; their scores are masked to -inf before use.
    auto issue_tile = [&](int t, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const int k0 = t * KB;
        if (FA2_POISON_LDS) {
            typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) u32x4p lds_u32x4;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const uint32_t dst = lds_base + 2u * (i * NW + wave) * 512 + 16u * lane;
                const u32x4p nan4 = u32x4p{~0u, ~0u, ~0u, ~0u};
                *(lds_u32x4*)(uintptr_t)(dst + 2u * (ST * 2 + 0) * LTILE) = nan4;
                *(lds_u32x4*)(uintptr_t)(dst + 2u * (ST * 2 + 1) * LTILE) = nan4;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if (k0 + KB <= len) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const long long rows = (long long)k0 + i * ROWS_PER_LOAD;
                const uint32_t dst = lds_base + 2u * (i * NW + wave) * 512;
                dma_16B_s(Kh + rows * kv_sr, offK, dst + 2u * (ST * 2 + 0) * LTILE);
                dma_16B_s(Vh + rows * kv_sr, offV, dst + 2u * (ST * 2 + 1) * LTILE);
            }
        } else {
            // (opaque copies of the lane offsets: otherwise the compiler keeps
            // the per-lane 64-bit addresses Kh + offK, Vh + offV live across
            // the whole scan for this one stage)
            uint32_t oK = offK, oV = offV;
            asm volatile("" : "+v"(oK), "+v"(oV));
            // The lane's load row again, from a lane index the compiler cannot
            // hoist: otherwise it keeps row0 live across the scan for this one
            // stage and spills it.
            int ln;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            const int r0 = (wave * 64 + ln) / CPR;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int r = r0 + i * ROWS_PER_LOAD;
                const long long shift = (long long)(min(k0 + r, len - 1) - r0) * kv_sr;
                const uint32_t dst = lds_base + 2u * (i * NW + wave) * 512;
                dma_16B_v((const char*)(Kh + shift) + oK, dst + 2u * (ST * 2 + 0) * LTILE);
                dma_16B_v((const char*)(Vh + shift) + oV, dst + 2u * (ST * 2 + 1) * LTILE);
            }
        }
    };

    issue_tile(t_begin, Int<0>{});

    if constexpr (MF32) {
    // ---- the 32x32x16 path (D = 64 without dropout) ----
    // Lane layouts of v_mfma_f32_32x32x16_f16 (32x16 A, 16x32 B, 32x32 C):
    //   A[i][k] -> lane i + 32*(k/8), element k%8
    //   B[k][j] -> lane j + 32*(k/8), element k%8
    //   C[i][j] -> lane j + 32*((i/4)%2), element i%4 + 4*(i/8)
    // With S^T = K Q^T a lane holds one query (lane%32) and, of each 32-key
    // block, keys 8t + 4h + e (h = lane/32) in element 4t + e: 32 scores per
    // lane per 64-key tile, two lanes (l, l^32) per query. For the PV product
    // over 16-key step w of a block, elements 8w .. 8w+7 of a lane are keys
    // {16w + 4h + 0..3, 16w + 8 + 4h + 0..3}; taken in that order as the 8
    // k-values of the lane they are the B operand P^T directly, and the V^T A
    // operand uses the same key order (two transposing reads of 4 rows). Each
    // MFMA does twice the work of a 16x16x32 one for the same issue cost, which
    // the softmax's VALU work competes with.
    constexpr int DS = D / 16;     // k-steps of one 32x32x16 score block
    constexpr int NB32 = BN / 32;  // 32-key blocks per compute tile
    constexpr int DB32 = D / 32;   // 32-row blocks of O^T
    const int l32 = lane & 31, hh = lane >> 5;

    half8 qreg[DS];
    {
        const int row = min(qw0 + l32, len - 1);
#pragma unroll
        for (int st = 0; st < DS; ++st)
            qreg[st] = *reinterpret_cast<const half8*>(Qh + (long long)row * q_sr + 16 * st + 8 * hh);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // Q only (see the 16x16x32 path)

    f32x16 oacc[DB32];
#pragma unroll
    for (int db = 0; db < DB32; ++db) oacc[db] = f32x16{};
    float mc_run = kMaxInit, l_run = 0.f;
    // Row sums on the matrix unit: a 16x16x32 MFMA whose B operand is one P^T
    // fragment of this layout. Its B[k][j] sits in lane j + 16*(k/8), so k-group
    // G = k/8 holds query j + 16*(G%2) (of half G/2). An A operand of ones where
    // (k/8)%2 == i%2 and zeros elsewhere makes output row i the sum over query
    // j + 16*(i%2); in the 16x16 C layout lane L finds its own query's sum in
    // element (L/16)%2. A[i][k] sits in lane i + 16*(k/8): each lane holds 8
    // equal values, ones where (L/16)%2 == L%2.
    half8 kSumSel;
    {
        const uint32_t v = (((lane >> 4) ^ lane) & 1) ? 0u : 0x3c003c00u;
        typedef uint32_t u32x4w __attribute__((ext_vector_type(4)));
        kSumSel = __builtin_bit_cast(half8, u32x4w{v, v, v, v});
    }
    bool fresh = true;

    // Tile-independent LDS read offsets (bytes). K: row l32 of a block, logical
    // chunk 2*step + h; the step only flips bits the row term leaves clear:
    // offset(step) = rdK ^ (step << 5). V: source lane (column half G, index i)
    // of a transposing read points at row 4h + i/4 (+8 for the second read) and
    // columns 16G + 4(i%4) .. +3; the column block db flips chunk bit 2:
    // offset(db) = rdV ^ (db << 6).
    const uint32_t rdK = 2u * (l32 * D) + 16u * (hh ^ swz_k<D>(l32));
    const uint32_t rdV = [&] {
        const int i = lane & 15, G = (lane >> 4) & 1;
        const int r = 4 * hh + (i >> 2);
        return 2u * (r * D) + 16u * ((2 * G + ((i & 3) >> 1)) ^ swz_v32(r)) + 8u * (i & 1);
    }();

    auto compute_tile32 = [&](const int k0, const char* const ldsK, const char* const ldsV)
                              __attribute__((always_inline)) {
        uint32_t rk = rdK, rv = rdV;
        asm volatile("" : "+v"(rk), "+v"(rv));

        // ---- S^T = K Q^T ----
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(FA2_PRIO_QK);
        f32x16 sacc[NB32];
#pragma unroll
        for (int st = 0; st < DS; ++st)
#pragma unroll
            for (int kb = 0; kb < NB32; ++kb) {
                const half8 ka = *reinterpret_cast<const half8*>(ldsK + (rk ^ (st << 5)) + kb * 32 * D * 2);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qreg[st], st == 0 ? f32x16{} : sacc[kb],
                                                                  0, 0, 0);
            }
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(FA2_PRIO_SM);

        // ---- masks ----
        bool need_mask = k0 + BN > len;
        if (MASK == kCausal) need_mask |= k0 + BN - 1 > qw0;
        if (MASK == kWindow) need_mask |= (k0 < qw0 + QW - 1 - a.wl) || (k0 + BN - 1 > qw0 + a.wr);
        if (need_mask) {
            // admissible keys [lo, hi) per row, as in the 16x16x32 path
            const int qrow = qw0 + l32;
            const int base = k0 + 4 * hh;
            int hi = len;
            if (MASK == kCausal) hi = min(hi, qrow + 1);
            if (MASK == kWindow) hi = min(hi, qrow + a.wr + 1);
            hi -= base;
            const int lo = MASK == kWindow ? max(0, qrow - a.wl) - base : 0;
            const uint32_t width = (uint32_t)max(hi - lo, 0);
#pragma unroll
            for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int off = 32 * kb + 8 * t + e;
                        const bool keep = MASK == kWindow ? (uint32_t)(off - lo) < width : off < hi;
                        if (!keep) sacc[kb][4 * t + e] = -INFINITY;
                    }
        }

        // ---- online softmax, the same lazy reference as the 16x16x32 path ----
        half8 pb[NB32][2];
        float rs;
        auto exponentiate = [&]() __attribute__((always_inline)) {
            const float mc = mc_run;
#pragma unroll
            for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    half2 h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * w + 2 * e], a.c, -mc));
                        const float p1 =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * w + 2 * e + 1], a.c, -mc));
                        h[e] = half2{(_Float16)p0, (_Float16)p1};
                    }
                    pb[kb][w] = half8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
                }
            f32x4 ls = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
                for (int w = 0; w < 2; ++w) ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(kSumSel, pb[kb][w], ls, 0, 0, 0);
            rs = (lane & 16) ? ls[1] : ls[0];
        };
        bool move_ref = fresh;
        if (!move_ref) {
            exponentiate();
            // An overflowed p makes its query's sum inf and, through the zero
            // weights of the selecting operand (0 * inf), the other query's sum
            // NaN. Compared as unsigned integers (the sums are never negative)
            // both are above the bound, a test that does not depend on NaN
            // semantics.
            move_ref = __builtin_amdgcn_ballot_w64(__float_as_uint(rs) >= __float_as_uint(kSpeculateLimit)) != 0;
        }
        if (move_ref) {
            float m0 = fmaxf(sacc[0][0], sacc[0][1]);
            float m1 = fmaxf(sacc[0][2], sacc[0][3]);
#pragma unroll
            for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
                for (int e = (kb == 0 ? 4 : 0); e < 16; e += 2) {
                    m0 = fmaxf(m0, sacc[kb][e]);
                    m1 = fmaxf(m1, sacc[kb][e + 1]);
                }
            const float m_new = fmaxf(mc_run, __builtin_fmaf(max_xor32(fmaxf(m0, m1)), a.c, kRefHeadroom));
            const float alpha = __builtin_amdgcn_exp2f(mc_run - m_new);
            mc_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB32; ++db) oacc[db] *= alpha;
            exponentiate();
        }
        fresh = false;
        l_run += rs;

        // ---- O^T += V^T P^T ----
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(FA2_PRIO_PV);
#pragma unroll
        for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
            for (int w = 0; w < 2; ++w)
#pragma unroll
                for (int db = 0; db < DB32; ++db) {
                    const char* p0 = ldsV + (rv ^ (db << 6)) + (32 * kb + 16 * w) * D * 2;
                    const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
                    const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * D * 2));
                    const half4 h0 = __builtin_bit_cast(half4, t0);
                    const half4 h1 = __builtin_bit_cast(half4, t1);
                    const half8 va = half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kb][w], oacc[db], 0, 0, 0);
                }
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(0);
    };

    auto tile_step32 = [&](int t, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < t_end) issue_tile(t + 1, Int<1 - ST>{});
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            const int k0 = t * KB + j * BN;
            if (k0 >= kend) break;
            if (MASK == kCausal && k0 > qw0 + QW - 1) break;
            if (MASK == kWindow) {
                if (k0 > qw0 + QW - 1 + a.wr) break;
                if (k0 + BN - 1 < qw0 - a.wl) continue;
            }
            compute_tile32(k0, reinterpret_cast<const char*>(smem) + 2 * ((ST * 2 + 0) * LTILE + j * TILE),
                           reinterpret_cast<const char*>(smem) + 2 * ((ST * 2 + 1) * LTILE + j * TILE));
        }
    };
    for (int t = t_begin; t < t_end; t += 2) {
        tile_step32(t, Int<0>{});
        if (t + 1 < t_end) tile_step32(t + 1, Int<1>{});
    }

    // ---- epilogue: O = o / l in fp16, LSE = scale*m + ln(l) ----
    _Float16* __restrict__ Oh = a.o + b * a.q_sb + h * a.q_sh + (long long)start * q_sr;
    float* __restrict__ Lh = a.lse + b * a.l_sb + h * a.l_sh + start;
    const float inv = 1.0f / l_run;
    const int row = qw0 + l32;
    if (row < len) {
#pragma unroll
        for (int db = 0; db < DB32; ++db)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x16 ov = oacc[db];
                const half4 hv = half4{(_Float16)(ov[4 * t] * inv), (_Float16)(ov[4 * t + 1] * inv),
                                       (_Float16)(ov[4 * t + 2] * inv), (_Float16)(ov[4 * t + 3] * inv)};
                *reinterpret_cast<half4*>(Oh + (long long)row * q_sr + 32 * db + 8 * t + 4 * hh) = hv;
            }
        if (hh == 0) Lh[row] = (mc_run + log2f(l_run)) * kLn2;
    }
    } else {  // ---- the 16x16x32 path ----

    // Q^T as the B operand of the score MFMA, kept in registers for the whole scan.
    // Rows past the end are clamped (their results are never stored).
    half8 qreg[QB][DK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qw0 + 16 * qb + l16, len - 1);
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            qreg[qb][kk] = *reinterpret_cast<const half8*>(Qh + (long long)row * q_sr + 32 * kk + 8 * g);
    }
    // Wait for Q here with the compiler-visible s_waitcnt (vmcnt(0), expcnt and
    // lgkmcnt unconstrained): otherwise the compiler's wait for Q sits at its
    // first use inside the loop and, since vmcnt also counts the K/V loads of the
    // next tile, would stall on them every iteration.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    f32x4 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Per query row: the running reference in base-2 units (a score times c,
    // kept scaled so that the exponent needs one FMA and no multiply) and the
    // running sum l.
    float mc_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mc_run[qb] = kMaxInit;
        l_run[qb] = 0.f;
    }
    const half2 kOnes2 = half2{(_Float16)1.0f, (_Float16)1.0f};
    // All-ones MFMA operand of the matrix-unit row sums, kept live at D=64.
    constexpr bool KEEP_ONES = ROWSUM_MFMA && D == 64;
    half8 kOnesKeep = half8{};
    if (KEEP_ONES) {
        uint32_t o2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(o2[i]));
        typedef uint32_t u32x4w __attribute__((ext_vector_type(4)));
        kOnesKeep = __builtin_bit_cast(half8, u32x4w{o2[0], o2[1], o2[2], o2[3]});
    }
    bool fresh = true;  // no tile computed by this wave yet

    // LDS read offsets (bytes) that do not depend on the tile (lds_read_bases):
    //   offset(K, kk) = rdK0 ^ (kk << 6),   offset(V, db) = rdV0 ^ (db << 5).
    uint32_t rdK0, rdV0;
    lds_read_bases<D>(lane, rdK0, rdV0);

    // Per-tile register arrays: the S^T accumulators and the fp16 P^T operands.
    typedef f32x4 SAccT[QB][NKB];
    typedef half8 PBT[QB][NKC];

    // ---- S^T = K Q^T on MFMA for the compute tile at k0 (K at ldsK), then the
    // masks: keys past the end, after the query (causal), outside the window
    // (local) ----
    auto scores = [&](const int k0, const char* const ldsK, SAccT& sacc) __attribute__((always_inline)) {
        // The per-k-step offsets are derived from the base inside the tile; the
        // empty asm keeps the compiler from hoisting them out of the loop into
        // registers of their own.
        uint32_t rk = rdK0;
        asm volatile("" : "+v"(rk));
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(FA2_PRIO_QK);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // The k-steps of one 16-key block accumulate into the same registers;
        // FA2_QK_GROUP blocks are interleaved so that dependent MFMAs are
        // 2*FA2_QK_GROUP-1 independent ones apart.
#pragma unroll
        for (int kb0 = 0; kb0 < NKB; kb0 += FA2_QK_GROUP) {
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
#pragma unroll
                for (int kb = kb0; kb < kb0 + FA2_QK_GROUP; ++kb) {
                    const half8 ka = *reinterpret_cast<const half8*>(ldsK + (rk ^ (kk << 6)) + kb * 16 * D * 2);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qreg[qb][kk], sacc[qb][kb], 0, 0, 0);
                }
            }
        }
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(FA2_PRIO_SM);

        bool need_mask = k0 + BN > len;
        if (MASK == kCausal) need_mask |= k0 + BN - 1 > qw0;
        if (MASK == kWindow) need_mask |= (k0 < qw0 + QW - 1 - a.wl) || (k0 + BN - 1 > qw0 + a.wr);
        if (need_mask) {
            // The admissible keys of a row are one range, [lo, hi): hi =
            // min(len, i+1) causal, min(len, i+wr+1) windowed, len otherwise;
            // lo = max(0, i-wl) windowed, else 0. Element (kb, e) of a lane is
            // key k0 + 4g + (16kb + e), so per lane the range shifts by
            // k0 + 4g once and each element compares its constant offset:
            // one compare (two for a window, as one unsigned range test) and
            // one select per score.
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qrow = qw0 + 16 * qb + l16;
                const int base = k0 + 4 * g;
                int hi = len;
                if (MASK == kCausal) hi = min(hi, qrow + 1);
                if (MASK == kWindow) hi = min(hi, qrow + a.wr + 1);
                hi -= base;
                const int lo = MASK == kWindow ? max(0, qrow - a.wl) - base : 0;
                const uint32_t width = (uint32_t)max(hi - lo, 0);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int off = 16 * kb + e;
                        const bool keep = MASK == kWindow ? (uint32_t)(off - lo) < width : off < hi;
                        if (!keep) sacc[qb][kb][e] = -INFINITY;
                    }
            }
        }
    };

    // ---- online softmax update ----
    // Probabilities are taken against the running reference m (held as
    // mc_run = m*c): p = 2^(s*c - m*c). l and o always use the same
    // reference per row, so O = o/l and LSE = scale*m + ln l hold for any
    // reference; it only has to keep every p representable in fp16. The
    // common path therefore skips the row max: it exponentiates the tile
    // against the current reference and accepts the result if the row
    // sums of the fp16 p (a lane's partial sums, or with the matrix-unit
    // sums the tile's full row sums) stay below 2^15, so no p overflowed.
    // A wave's first tile, or a tile that fails the check for any of its
    // rows, takes the row max (combined over the 4 lanes of a query),
    // moves the reference to max(m, max + kRefHeadroom), rescales o and l by
    // alpha = 2^((m_old - m_new)*c) and exponentiates again: the update
    // of the online softmax.

    // p of 32-key chunk kc (16-key blocks 2kc, 2kc+1) of query block qb, as
    // the fp16 B operand of the PV product, and its partial row sum (over
    // the fp16 values, before dropout: the softmax normaliser counts every
    // admissible key).
    auto exp_chunk = [&](const SAccT& sacc, PBT& pb, int qb, int kc, float& rsum) __attribute__((always_inline)) {
        const float mc = mc_run[qb];
        const f32x4 lo = sacc[qb][2 * kc], hi = sacc[qb][2 * kc + 1];
        half2 h[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(lo[2 * e], a.c, -mc));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(lo[2 * e + 1], a.c, -mc));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(hi[2 * e], a.c, -mc));
            const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(hi[2 * e + 1], a.c, -mc));
            h[e] = half2{(_Float16)p0, (_Float16)p1};
            h[2 + e] = half2{(_Float16)p2, (_Float16)p3};
        }
        if (!ROWSUM_MFMA) {
#pragma unroll
            for (int e = 0; e < 4; ++e) rsum = __builtin_amdgcn_fdot2(h[e], kOnes2, rsum, false);
        }
        pb[qb][kc] = half8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    };
    // Row max over 16-key blocks kb0 .. kb1-1, combined over the 4 lanes of a query.
    auto row_max = [&](const SAccT& sacc, int qb, int kb0, int kb1) __attribute__((always_inline)) {
        float a0 = fmaxf(sacc[qb][kb0][0], sacc[qb][kb0][1]);
        float a1 = fmaxf(sacc[qb][kb0][2], sacc[qb][kb0][3]);
        for (int kb = kb0 + 1; kb < kb1; ++kb) {
            a0 = fmaxf(a0, fmaxf(sacc[qb][kb][0], sacc[qb][kb][1]));
            a1 = fmaxf(a1, fmaxf(sacc[qb][kb][2], sacc[qb][kb][3]));
        }
        return max_xor32(max_xor16(fmaxf(a0, a1)));
    };
    // Move the reference of query block qb up to kRefHeadroom above the raw
    // score mx (if higher), rescaling o and l.
    auto move_reference = [&](int qb, float mx) __attribute__((always_inline)) {
        const float m_new = fmaxf(mc_run[qb], __builtin_fmaf(mx, a.c, kRefHeadroom));
        const float alpha = __builtin_amdgcn_exp2f(mc_run[qb] - m_new);
        mc_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
    };

    // ---- dropout on P: zero the probabilities of dropped keys ----
    // Key j of query row i (both within the sequence) of head (b, h) takes
    // 16-bit draw j%8 of Philox4x32-10 at counter (j/8, i, b*H + h, offset)
    // under key (seed_lo, seed_hi) (draw t = bits 16*(t%2) of word t/2),
    // and is kept when the draw is >= drop_thr. A lane holds keys
    // 4g..4g+3 of the two 16-key blocks of chunk kc; lanes g and g^1 (the
    // two 16-lane rows a v_permlane16_swap pairs) need the same two groups
    // of 8 keys, g even the low four draws and g odd the high four. So
    // each lane computes one group (g even that of the first block, g odd
    // that of the second) and two swaps hand each lane the other lane's
    // words it needs. Kept probabilities are scaled by 1/(1-p) in the
    // epilogue.
    auto drop_chunk = [&](const int k0, PBT& pb, int kc) __attribute__((always_inline)) {
        // The lane's part of the counter, through an opaque copy: otherwise
        // the compiler keeps one sum per chunk position live across the scan
        // and spills them (not needed in the half-height causal instance,
        // which stays within its registers and runs 1 % faster without it).
        uint32_t gl = 2u * (uint32_t)(g & 1) + (uint32_t)(g >> 1);
        if (!(NW == 4 && MASK == kCausal)) asm volatile("" : "+v"(gl));
        uint32_t group = (uint32_t)((k0 + 32 * kc) >> 3) + gl;
        // Opaque to the optimiser: the counter grows linearly with the
        // tile, and loop strength reduction otherwise keeps the first
        // round's 64-bit product for every chunk position of a stage live
        // across the scan (16 VGPRs), which spills.
        asm volatile("" : "+v"(group));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint32_t qrow = (uint32_t)(qw0 + 16 * qb + l16);
            const U32x4 r = philox4x32_10(group, qrow, (uint32_t)bh, a.offset, a.seed_lo, a.seed_hi);
            // after the swaps: x = this lane's two words for the first
            // block, y = for the second
            const auto s0 = __builtin_amdgcn_permlane16_swap(r.w[0], r.w[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(r.w[1], r.w[3], false, false);
            const uint32_t w[4] = {s0[0], s1[0], s0[1], s1[1]};
            // Keep mask per 16-bit half, 0xFFFF for draw >= drop_thr and 0
            // otherwise, in three packed 16-bit integer ops per word:
            // sat(thr - draw) is 0 exactly for kept keys, min(., 1) - 1
            // (wrapping) maps 0 to 0xFFFF and 1 to 0. drop_thr <= 0xFFFF, and
            // drop_thr = 0 keeps every key.
            const uint32_t thr2 = a.drop_thr * 0x00010001u;
            const uint32_t one2 = 0x00010001u;
            uint32_t m[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t over, m01;
                asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(over) : "v"(thr2), "v"(w[e]));
                asm("v_pk_min_u16 %0, %1, %2" : "=v"(m01) : "v"(over), "v"(one2));
                asm("v_pk_sub_u16 %0, %1, %2" : "=v"(m[e]) : "v"(m01), "v"(one2));
            }
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            u32x4v bits = __builtin_bit_cast(u32x4v, pb[qb][kc]);
            bits &= u32x4v{m[0], m[1], m[2], m[3]};
            pb[qb][kc] = __builtin_bit_cast(half8, bits);
        }
    };

    // ---- O^T += V^T P^T on MFMA ----
    // Source lane l16 of group g points at row 4g + l16/4 (+16 for the second
    // half) and columns 16*db + 4*(l16%4) .. +3; the transposing read returns
    // V[32kc + 4g + e][16db + l16] in element e.
    auto read_v = [&](const char* const ldsV, uint32_t rv, int kc, int db) __attribute__((always_inline)) {
        const char* p0 = ldsV + (rv ^ (db << 5)) + kc * 32 * D * 2;
        const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
        const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * D * 2));
        const half4 h0 = __builtin_bit_cast(half4, t0);
        const half4 h1 = __builtin_bit_cast(half4, t1);
        return half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
    };
    // At D=128 (2 waves per SIMD, registers to spare) the V fragments of the
    // first chunk are read before the softmax, so that their LDS latency hides
    // under its VALU work. At D=64 the registers are not there.
    constexpr int VPRE = (D == 128) ? DB : 0;
    typedef half8 VPreT[VPRE > 0 ? VPRE : 1];
    auto pv_tile = [&](const char* const ldsV, uint32_t rv, const PBT& pb, const VPreT& vpre)
                       __attribute__((always_inline)) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const half8 va = (kc == 0 && db < VPRE) ? vpre[db] : read_v(ldsV, rv, kc, db);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[qb][kc], oacc[db][qb], 0, 0, 0);
            }
    };

    // Exponentiate the whole tile against the current reference; rs gets the
    // row sums used by the check and added to l.
    auto exponentiate = [&](const SAccT& sacc, PBT& pb, float (&rs)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            rs[qb] = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) exp_chunk(sacc, pb, qb, kc, rs[qb]);
        }
        if (ROWSUM_MFMA) {
            // the tile's full row sums on the matrix unit (each lane gets
            // its query's sum over all BN keys): an MFMA with an all-ones
            // A operand sums the B operand (P^T) over its 32 keys. At D=64
            // the constant stays in registers for the whole scan; at D=128
            // it is rebuilt here with volatile moves, which measured
            // faster there than keeping it live.
            half8 kOnes8 = kOnesKeep;
            if (!KEEP_ONES) {
                uint32_t one2[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(one2[i]));
                typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
                kOnes8 = __builtin_bit_cast(half8, u32x4v{one2[0], one2[1], one2[2], one2[3]});
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                f32x4 ls = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
                    ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(kOnes8, pb[qb][kc], ls, 0, 0, 0);
                rs[qb] = ls[0];
            }
        }
    };
    // True (on every lane) when a row sum of the speculative exponentiation
    // reached 2^15, i.e. some p may have overflowed fp16.
    auto overflowed = [&](const float (&rs)[QB]) __attribute__((always_inline)) {
        bool over = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) over |= !(rs[qb] < kSpeculateLimit);
        return __builtin_amdgcn_ballot_w64(over) != 0;  // wave-uniform
    };
    auto rebase = [&](const SAccT& sacc) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) move_reference(qb, row_max(sacc, qb, 0, NKB));
    };

    // One compute tile: keys k0 .. k0+BN-1, K and V at the given LDS addresses.
    auto compute_tile = [&](const int k0, const char* const ldsK, const char* const ldsV)
                            __attribute__((always_inline)) {
        // the per-column-block V offsets, derived inside the tile like the K ones
        uint32_t rv = rdV0;
        asm volatile("" : "+v"(rv));
        SAccT sacc;
        scores(k0, ldsK, sacc);
        VPreT vpre;
#pragma unroll
        for (int i = 0; i < VPRE; ++i) vpre[i] = read_v(ldsV, rv, 0, i);
        PBT pb;
        float rs[QB];
        bool move_ref = fresh;
        if (!move_ref) {
            exponentiate(sacc, pb, rs);
            move_ref = overflowed(rs);
        }
        if (move_ref) {
            rebase(sacc);
            exponentiate(sacc, pb, rs);
        }
        fresh = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
        if (DROP) {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) drop_chunk(k0, pb, kc);
        }
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(FA2_PRIO_PV);
        pv_tile(ldsV, rv, pb, vpre);
        if (FA2_SETPRIO) __builtin_amdgcn_s_setprio(0);
    };

    // One step of the scan over ring stage t (SUB compute tiles) held in stage ST.
    auto tile_step = [&](int t, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        // Stage t is resident for every wave (each waits for its own loads, then
        // the barrier), and every wave has finished reading the other stage
        // (stage t-1), which the next loads overwrite.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < t_end) issue_tile(t + 1, Int<1 - ST>{});
        auto ldsK = [&](int j) { return reinterpret_cast<const char*>(smem) + 2 * ((ST * 2 + 0) * LTILE + j * TILE); };
        auto ldsV = [&](int j) { return reinterpret_cast<const char*>(smem) + 2 * ((ST * 2 + 1) * LTILE + j * TILE); };
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            const int k0 = t * KB + j * BN;
            if (k0 >= kend) break;                                 // past the keys needed
            if (MASK == kCausal && k0 > qw0 + QW - 1) break;       // above this wave's diagonal
            if (MASK == kWindow) {
                if (k0 > qw0 + QW - 1 + a.wr) break;               // right of this wave's band
                if (k0 + BN - 1 < qw0 - a.wl) continue;            // left of this wave's band
            }
            compute_tile(k0, ldsK(j), ldsV(j));
        }
    };

    // The ring stage alternates with the tile index; stepping two tiles per
    // iteration makes it a compile-time constant, so LDS offsets are immediates.
    for (int t = t_begin; t < t_end; t += 2) {
        tile_step(t, Int<0>{});
        if (t + 1 < t_end) tile_step(t + 1, Int<1>{});
    }

    // ---- epilogue: O = o / l in fp16, LSE = scale*m + ln(l) ----
    _Float16* __restrict__ Oh = a.o + b * a.q_sb + h * a.q_sh + (long long)start * q_sr;
    float* __restrict__ Lh = a.lse + b * a.l_sb + h * a.l_sh + start;
    // The lane's row and column terms, derived again here from an opaque copy
    // of the lane index: otherwise the compiler keeps them live across the
    // scan and, at the 128-register budget, spills one to scratch.
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int l16e = lane_e & 15, ge = lane_e >> 4;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        // l_run holds per-lane partial sums (4 lanes per query) unless the row
        // sums come from the matrix unit, where every lane has the full sum.
        float lt = l_run[qb];
        if (!ROWSUM_MFMA) lt = sum_xor32(sum_xor16(lt));
        const float inv = (DROP ? a.out_scale : 1.0f) / lt;
        const int row = qw0 + 16 * qb + l16e;
        if (row < len) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4 ov = oacc[db][qb];
                const half4 hv = half4{(_Float16)(ov[0] * inv), (_Float16)(ov[1] * inv),
                                       (_Float16)(ov[2] * inv), (_Float16)(ov[3] * inv)};
                *reinterpret_cast<half4*>(Oh + (long long)row * q_sr + 16 * db + 4 * ge) = hv;
            }
            if (ge == 0) Lh[row] = (mc_run[qb] + log2f(lt)) * kLn2;
        }
    }
    }  // the 16x16x32 path
}

// Tile shapes per head dimension: <D, 16-query blocks per wave, waves, keys per
// compute tile, compute tiles per ring stage>. The defaults can be overridden at
// build time to compare tilings.
#ifndef FA2_D64_QB
#define FA2_D64_QB 2
#endif
#ifndef FA2_D64_NW
#define FA2_D64_NW 8
#endif
#ifndef FA2_D64_BN
#define FA2_D64_BN 64
#endif
#ifndef FA2_D128_QB
#define FA2_D128_QB 2
#endif
#ifndef FA2_D128_NW
#define FA2_D128_NW 8
#endif
#ifndef FA2_D128_BN
#define FA2_D128_BN 64
#endif
#ifndef FA2_D64_SUB
#define FA2_D64_SUB 2
#endif
// MFMA shape of the D = 64 instances without dropout: 16 (16x16x32) or 32 (32x32x16)
#ifndef FA2_D64_MF
#define FA2_D64_MF 16
#endif
#ifndef FA2_D128_SUB
#define FA2_D128_SUB 2
#endif
using Shape64 = Shape<64, FA2_D64_QB, FA2_D64_NW, FA2_D64_BN, FA2_D64_SUB, FA2_D64_MF>;
using Shape128 = Shape<128, FA2_D128_QB, FA2_D128_NW, FA2_D128_BN, FA2_D128_SUB>;
// Half-height workgroups (4 waves, 128 query rows, one compute tile per ring
// stage) for causal launches whose full-height grid fits in one round of
// resident workgroups: there every workgroup starts at once and the launch
// lasts as long as its heaviest (diagonal-most) workgroup, which halving the
// workgroup height halves. Larger causal grids are balanced by the
// heaviest-first order; they keep the full-height tiles unless the sequences
// are short (causal_half_height).
using Shape64c = Shape<64, FA2_D64_QB, 4, FA2_D64_BN, 1, FA2_D64_MF>;
using Shape128c = Shape<128, FA2_D128_QB, 4, FA2_D128_BN, 1>;

constexpr int kCUs = 256;                 // MI355X compute units
constexpr int kLdsPerCU = 160 * 1024;     // LDS bytes per compute unit

// Workgroups of shape SH resident per compute unit (LDS and register limits).
template <class SH>
constexpr int wg_per_cu() {
    return (kLdsPerCU / SH::LDS_BYTES) < (SH::WAVES_PER_SIMD * 4 / SH::NW) ? (kLdsPerCU / SH::LDS_BYTES)
                                                                           : (SH::WAVES_PER_SIMD * 4 / SH::NW);
}
#ifndef FA2_SMALL_CAUSAL
#define FA2_SMALL_CAUSAL 1
#endif
template <class SH>
bool fits_one_round(long long units, int S) {
    return FA2_SMALL_CAUSAL && units * ((S + SH::BM - 1) / SH::BM) <= (long long)kCUs * wg_per_cu<SH>();
}
// Dense causal launches run half-height workgroups when the full-height grid
// fits in one round (above), and also when the sequences are short: the 8
// waves of a full-height workgroup reach their diagonals up to 224 keys apart,
// and over a short causal scan the waves that finish first wait at the shared
// barriers; half the height halves that spread. Measured on one GPU, half-height
// was 3-9 % faster for S from 1000 to 3584 at D = 64 and 1-4 % faster for
// S <= 1024 at D = 128, about even at S = 4096 (D = 64) and S = 2048
// (D = 128), and 1-4 % slower for longer sequences, where the full height's
// two compute tiles per barrier win.
constexpr int kShortCausal64 = 4095;
constexpr int kShortCausal128 = 1024;
template <class SH>
bool causal_half_height(long long units, int S) {
    return fits_one_round<SH>(units, S) ||
           (FA2_SMALL_CAUSAL && S <= (SH::D == 64 ? kShortCausal64 : kShortCausal128));
}
// Other dense launches (unmasked or windowed) whose full-height grid is
// smaller than one round of resident workgroups leave compute units short of
// work: half the height doubles the workgroups. Measured on one GPU, unmasked:
// +24-25 % at 64-128 full-height workgroups and +8 % at 384 (D = 64), +19 % at
// 128 (D = 128), even at 256 (D = 64), and 3.5-6 % slower once the full-height
// grid fills a round; windowed grids of 256 full-height workgroups +2-5 %.
template <class SH>
bool plain_half_height(long long units, int S) {
    return FA2_SMALL_CAUSAL && units * ((S + SH::BM - 1) / SH::BM) < (long long)kCUs * wg_per_cu<SH>();
}

constexpr int kMaxDevices = 64;

template <class SH, int MASK, bool DROP>
hipError_t launch_shape(const LaunchArgs& a, const KernelArgs& k, hipStream_t stream) {
    auto kern = fa2_fwd_kernel<SH, MASK, DROP>;
    if (SH::LDS_BYTES > 65536) {
        // Opt in to more than 64 KiB of dynamic LDS, once per device.
        static std::atomic<bool> attr_set[kMaxDevices];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
        if (dev < 0 || dev >= kMaxDevices || !attr_set[dev].load(std::memory_order_acquire)) {
            hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               SH::LDS_BYTES);
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < kMaxDevices) attr_set[dev].store(true, std::memory_order_release);
        }
    }
    // One workgroup per (sequence, head, query tile). A 1-D grid keeps
    // blocks * threads below 2^32; beyond that the id is split over (x, y) with
    // x a multiple of 8 so that id mod 8 still names the XCD.
    constexpr unsigned kMaxX = 1u << 22;
    const unsigned nb = (unsigned)k.nblocks;
    const dim3 grid(nb <= kMaxX ? nb : kMaxX, nb <= kMaxX ? 1u : (nb + kMaxX - 1) / kMaxX);
    // hipLaunchKernel returns this launch's own status (an error left behind by
    // an earlier, unrelated runtime call of the caller is not reported as ours).
    KernelArgs karg = k;
    void* params[] = {&karg};
    (void)a;
    return hipLaunchKernel((const void*)kern, grid, dim3(SH::THREADS), params, SH::LDS_BYTES, stream);
}

template <class SH>
hipError_t launch_d(const LaunchArgs& a, hipStream_t stream) {
    KernelArgs k{};
    k.q = static_cast<const _Float16*>(a.q);
    k.k = static_cast<const _Float16*>(a.k);
    k.v = static_cast<const _Float16*>(a.v);
    k.o = static_cast<_Float16*>(a.o);
    k.lse = a.lse;
    k.cu = a.cu_seqlens;
    const long long D = a.D;
    if (a.cu_seqlens) {
        // packed [total, H, D] / [total, H_kv, D]; lse [H, total]
        k.q_sb = 0;
        k.q_sh = D;
        k.q_sr = (int)(a.H * D);
        k.kv_sb = 0;
        k.kv_sh = D;
        k.kv_sr = (int)(a.H_kv * D);
        k.l_sb = 0;
        k.l_sh = a.total;
    } else {
        // dense [B, H, S, D] / [B, H_kv, S, D]; lse [B, H, S]
        k.q_sr = (int)D;
        k.q_sh = (long long)a.S * D;
        k.q_sb = (long long)a.H * k.q_sh;
        k.kv_sr = (int)D;
        k.kv_sh = (long long)a.S * D;
        k.kv_sb = (long long)a.H_kv * k.kv_sh;
        k.l_sh = a.S;
        k.l_sb = (long long)a.H * a.S;
    }
    k.S = a.S;
    k.total = a.total;
    k.H = a.H;
    k.group = a.H / a.H_kv;
    k.BH = a.B * a.H;
    k.BHkv = a.B * a.H_kv;
    k.nqt = (a.S + SH::BM - 1) / SH::BM;
    // in 64-bit: the argument checks bound it by 2^31 - 1 for every shape
    const long long nblocks = a.cu_seqlens ? (((long long)k.BHkv + 7) / 8) * 8 * k.nqt * k.group
                                           : (long long)k.BH * k.nqt;
    if (nblocks > 0x7fffffffll) return hipErrorInvalidConfiguration;
    k.nblocks = (int)nblocks;
    k.c = (float)((double)a.scale * kLog2e);
    // A dense grid that is resident in one round takes the serpentine causal order.
    k.serp = (!a.cu_seqlens && k.nblocks <= kCUs * wg_per_cu<SH>()) ? kCUs / 8 : 0;
    // Packed tables of up to 64 sequences (one per lane) are walked longest first.
    k.lpt = (a.cu_seqlens && a.B <= 64) ? 1 : 0;

    // Window: a negative or out-of-range side is unbounded (S keys).
    const bool left_open = a.window_left < 0 || a.window_left >= a.S;
    const bool right_open = a.window_right < 0 || a.window_right >= a.S;
    int mask = kWindow;
    if (left_open && right_open) mask = kNoMask;
    else if (left_open && a.window_right == 0) mask = kCausal;
    k.wl = left_open ? a.S : a.window_left;
    k.wr = right_open ? a.S : a.window_right;

    const bool drop = a.dropout_p > 0.0f;
    k.out_scale = drop ? (float)(1.0 / (1.0 - (double)a.dropout_p)) : 1.0f;
    k.drop_thr = drop_threshold(a.dropout_p);
    k.seed_lo = (uint32_t)a.seed;
    k.seed_hi = (uint32_t)(a.seed >> 32);
    k.offset = a.offset;

    if (drop) {
        if (mask == kNoMask) return launch_shape<SH, kNoMask, true>(a, k, stream);
        if (mask == kCausal) return launch_shape<SH, kCausal, true>(a, k, stream);
        return launch_shape<SH, kWindow, true>(a, k, stream);
    }
    if (mask == kNoMask) return launch_shape<SH, kNoMask, false>(a, k, stream);
    if (mask == kCausal) return launch_shape<SH, kCausal, false>(a, k, stream);
    return launch_shape<SH, kWindow, false>(a, k, stream);
}

}  // namespace

template <class SH>
TileShape describe() {
    return {SH::BM, SH::KB, SH::THREADS, SH::LDS_BYTES};
}

TileShape tile_shape(int D) { return D == 128 ? describe<Shape128>() : describe<Shape64>(); }

int min_rows_per_block(int D) {
    return D == 128 ? (Shape128::BM < Shape128c::BM ? Shape128::BM : Shape128c::BM)
                    : (Shape64::BM < Shape64c::BM ? Shape64::BM : Shape64c::BM);
}

// A dense launch is causal when the left side of the window is open and the
// right side is 0 (the rule launch_d applies).
static bool causal_window(int S, int wl, int wr) { return (wl < 0 || wl >= S) && wr == 0; }

// Whether a dense launch runs the half-height workgroups.
template <class SH>
bool dense_half_height(long long units, int S, int wl, int wr) {
    return causal_window(S, wl, wr) ? causal_half_height<SH>(units, S) : plain_half_height<SH>(units, S);
}

TileShape dense_tile_shape(int D, long long units, int S, int window_left, int window_right) {
    if (D == 128)
        return dense_half_height<Shape128>(units, S, window_left, window_right) ? describe<Shape128c>()
                                                                                 : describe<Shape128>();
    return dense_half_height<Shape64>(units, S, window_left, window_right) ? describe<Shape64c>() : describe<Shape64>();
}

uint32_t drop_threshold(float p) {
    if (!(p > 0.0f)) return 0u;
    const double t = std::floor((double)p * 65536.0);
    return t >= 65535.0 ? 0xFFFFu : (uint32_t)t;
}

// Packed causal batches take the half-height workgroups when their sequences
// are short on average (total rows / sequences below the dense threshold):
// 24 packed sequences of 64 to 4096 rows ran 5.5 % faster that way. (Windowed
// grids of a round or more keep the full height: 3.5-4.6 % slower with half
// height at B4 H8 S8192, windows (1024, 1024) and (1024, 0).)
template <class SH>
bool packed_half_height(const LaunchArgs& a) {
    return FA2_SMALL_CAUSAL && (long long)a.total <= (long long)a.B * (SH::D == 64 ? kShortCausal64 : kShortCausal128);
}

hipError_t launch_forward(const LaunchArgs& a, hipStream_t stream) {
    const long long units = (long long)a.B * a.H;
    const bool causal = causal_window(a.S, a.window_left, a.window_right);
    if (a.D == 64) {
        const bool half = a.cu_seqlens ? causal && packed_half_height<Shape64>(a)
                                       : dense_half_height<Shape64>(units, a.S, a.window_left, a.window_right);
        return half ? launch_d<Shape64c>(a, stream) : launch_d<Shape64>(a, stream);
    }
    const bool half = a.cu_seqlens ? causal && packed_half_height<Shape128>(a)
                                   : dense_half_height<Shape128>(units, a.S, a.window_left, a.window_right);
    return half ? launch_d<Shape128c>(a, stream) : launch_d<Shape128>(a, stream);
}

}  // namespace fa2
