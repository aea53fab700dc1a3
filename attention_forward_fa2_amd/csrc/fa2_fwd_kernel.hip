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
// gfx950 mapping (lane layouts measured on the device, see the design notes):
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
//   * The row max and the final row sum combine the 4 lanes that share a query
//     (lanes l, l^16, l^32, l^48) with v_permlane16_swap / v_permlane32_swap:
//     the reduction group follows the accumulator ownership (§"把 lane 公式真正写出来").
//   * K and V tiles go HBM -> LDS with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4, LDS destination = base + 16*lane) into a
//     two-stage ring (§"多 Stage 流水"); the tile for step t+1 is in flight while
//     step t computes. The XOR swizzle of 16-byte chunks is applied on the
//     source side because the LDS side of these loads is lane-linear.
//   * Softmax runs in base 2: the max is taken on raw scores, then
//     p = 2^(s*c - m*c) with c = scale*log2(e), one FMA and one v_exp_f32 per
//     score (§"沿 C fragment 做 Online Softmax", closing paragraph).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr double kLog2e = 1.44269504088896340736;
// Finite start value of the running max: exp2((m0 - m) * c) is exactly 0 for any
// real score m, and a row whose keys were all masked so far keeps alpha = 1, p = 0.
constexpr float kMaxInit = -1.0e30f;

template <int D_, int QB_, int NW_, int BN_>
struct Shape {
    static constexpr int D = D_;
    static constexpr int QB = QB_;            // 16-query blocks per wave
    static constexpr int NW = NW_;            // waves per workgroup
    static constexpr int BN = BN_;            // keys per tile
    static constexpr int QW = 16 * QB;        // query rows per wave
    static constexpr int BM = NW * QW;        // query rows per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int NKB = BN / 16;       // 16-key blocks per tile
    static constexpr int NKC = BN / 32;       // 32-key chunks per tile
    static constexpr int DK = D / 32;         // k-steps of one score MFMA block
    static constexpr int DB = D / 16;         // 16-wide column blocks of the output
    static constexpr int CPR = D / 8;         // 16-byte chunks per row
    static constexpr int TILE = BN * D;       // halves per K or V tile
    static constexpr int LOADS = TILE / 8 / 64 / NW;  // 16-byte loads per lane per tensor per tile
    static constexpr int LDS_BYTES = 2 /*stages*/ * 2 /*K,V*/ * TILE * 2;
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert((TILE / 8) % (64 * NW) == 0, "loads must divide evenly among lanes");
};

// XOR swizzles of the 16-byte chunk index within a row, chosen so that the 16
// rows read by one ds_read_b128 quarter-wave (K) and the 8 rows x 2 chunks read
// by one ds_read_b64_tr_b16 half-wave (V) land on distinct 16-byte bank groups
// of a 256-byte bank window.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
    return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
    return D == 64 ? (((row >> 1) & 3) << 1) : ((row & 7) << 1);
}

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

struct KernelArgs {
    const _Float16* q;
    const _Float16* k;
    const _Float16* v;
    _Float16* o;
    float* lse;
    int S;
    int BH;        // B*H
    int nqt;       // query tiles per head
    int nblocks;   // BH * nqt
    float c;       // scale * log2(e)
};

template <class SH, bool CAUSAL>
__global__ __launch_bounds__(SH::THREADS) void fa2_fwd_kernel(KernelArgs a) {
    constexpr int D = SH::D, QB = SH::QB, NW = SH::NW, BN = SH::BN, QW = SH::QW, BM = SH::BM;
    constexpr int NKB = SH::NKB, NKC = SH::NKC, DK = SH::DK, DB = SH::DB, CPR = SH::CPR;
    constexpr int TILE = SH::TILE;

    extern __shared__ __attribute__((aligned(16))) _Float16 smem[];
    // [stage][K | V][TILE]
    _Float16* const lds = smem;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;

    // Workgroup -> (head, query tile). Consecutive workgroup ids go round-robin
    // to the 8 XCDs; regroup them so each XCD gets a contiguous run of logical
    // ids, which keeps the query tiles of one head (and its K/V in L2) together.
    const int bid = blockIdx.x;
    const int per = a.nblocks >> 3, rem = a.nblocks & 7, xcd = bid & 7;
    const int logical = xcd * per + min(xcd, rem) + (bid >> 3);
    int bh, qt;
    if (CAUSAL) {  // heaviest query tiles (most key tiles) first
        qt = a.nqt - 1 - logical / a.BH;
        bh = logical % a.BH;
    } else {
        bh = logical / a.nqt;
        qt = logical % a.nqt;
    }

    const int S = a.S;
    const long long head = (long long)bh * S * D;
    const _Float16* __restrict__ Qh = a.q + head;
    const _Float16* __restrict__ Kh = a.k + head;
    const _Float16* __restrict__ Vh = a.v + head;
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * QW;

    // Q^T as the B operand of the score MFMA, kept in registers for the whole scan.
    // Rows past the end are clamped (their results are never stored).
    half8 qreg[QB][DK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qw0 + 16 * qb + l16, S - 1);
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            qreg[qb][kk] = *reinterpret_cast<const half8*>(Qh + (long long)row * D + 32 * kk + 8 * g);
    }

    f32x4 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = kMaxInit;
        l_run[qb] = 0.f;
    }

    int n_tiles = (S + BN - 1) / BN;
    if (CAUSAL) n_tiles = min(n_tiles, (min(q0 + BM, S) - 1) / BN + 1);

    // Issue the direct-to-LDS loads of K/V tile t into ring stage st. Lane `lane`
    // of load instruction `inst` fills LDS chunk inst*64+lane, i.e. row r and
    // physical chunk pc; it fetches the logical chunk pc ^ swz(r) of key row
    // k0 + r (clamped to S-1: such rows are masked to -inf before use).
    auto issue_tile = [&](int t, int st) {
        const int k0 = t * BN;
        _Float16* const ldsK = lds + (st * 2 + 0) * TILE;
        _Float16* const ldsV = lds + (st * 2 + 1) * TILE;
#pragma unroll
        for (int i = 0; i < SH::LOADS; ++i) {
            const int inst = i * NW + wave;
            const int c = inst * 64 + lane;
            const int r = c / CPR, pc = c % CPR;
            const long long grow = min(k0 + r, S - 1);
            const _Float16* srcK = Kh + grow * D + 8 * (pc ^ swz_k<D>(r));
            const _Float16* srcV = Vh + grow * D + 8 * (pc ^ swz_v<D>(r));
            __builtin_amdgcn_global_load_lds(srcK, (lds_void*)(ldsK + inst * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(srcV, (lds_void*)(ldsV + inst * 512), 16, 0, 0);
        }
    };

    issue_tile(0, 0);
    for (int t = 0; t < n_tiles; ++t) {
        const int st = t & 1;
        // Tile t is resident for every wave, and every wave has finished reading
        // stage st^1 (tile t-1), which the next loads overwrite.
        __syncthreads();
        if (t + 1 < n_tiles) issue_tile(t + 1, st ^ 1);

        const int k0 = t * BN;
        if (CAUSAL && k0 > qw0 + QW - 1) continue;  // tile lies above this wave's diagonal

        const _Float16* const ldsK = lds + (st * 2 + 0) * TILE;
        const _Float16* const ldsV = lds + (st * 2 + 1) * TILE;

        // ---- S^T = K Q^T on MFMA ----
        f32x4 sacc[QB][NKB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int r = 16 * kb + l16;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const int lc = 4 * kk + g;
                const half8 ka = *reinterpret_cast<const half8*>(ldsK + r * D + 8 * (lc ^ swz_k<D>(r)));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qreg[qb][kk], sacc[qb][kb], 0, 0, 0);
            }
        }

        // ---- masks: keys past the end, and keys after the query when causal ----
        const bool need_mask = (k0 + BN > S) || (CAUSAL && k0 + BN - 1 > qw0);
        if (need_mask) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qrow = qw0 + 16 * qb + l16;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = k0 + 16 * kb + 4 * g + e;
                        if (key >= S || (CAUSAL && key > qrow)) sacc[qb][kb][e] = -INFINITY;
                    }
            }
        }

        // ---- online softmax update ----
        half8 pb[QB][NKC];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = sacc[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[qb][kb][e]);
            mx = max_xor16(mx);
            mx = max_xor32(mx);
            const float m_new = fmaxf(m_run[qb], mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * a.c);
            const float mc = m_new * a.c;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][e], a.c, -mc));
                    sacc[qb][kb][e] = p;
                    rs += p;
                }
            l_run[qb] = l_run[qb] * alpha + rs;
            m_run[qb] = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const f32x4 lo = sacc[qb][2 * kc], hi = sacc[qb][2 * kc + 1];
                pb[qb][kc] = half8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                                   (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
            }
        }

        // ---- O^T += V^T P^T on MFMA ----
        // Source lane l16 of group g points at row 4g + l16/4 (+16 for the second
        // half) and columns 16*db + 4*(l16%4) .. +3; the transposing read returns
        // V[32kc + 4g + e][16db + l16] in element e.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int lc = 2 * db + ((l16 & 3) >> 1);
            const int within = 4 * (l16 & 1);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const int r0 = 32 * kc + 4 * g + (l16 >> 2);
                const int r1 = r0 + 16;
                const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(ldsV + r0 * D + 8 * (lc ^ swz_v<D>(r0)) + within));
                const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(ldsV + r1 * D + 8 * (lc ^ swz_v<D>(r1)) + within));
                const half4 h0 = __builtin_bit_cast(half4, t0);
                const half4 h1 = __builtin_bit_cast(half4, t1);
                const half8 va = half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[qb][kc], oacc[db][qb], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: O = o / l in fp16, LSE = scale*m + ln(l) ----
    _Float16* __restrict__ Oh = a.o + head;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float lt = sum_xor16(l_run[qb]);
        lt = sum_xor32(lt);
        const float inv = 1.0f / lt;
        const int row = qw0 + 16 * qb + l16;
        if (row < S) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4 ov = oacc[db][qb];
                const half4 h = half4{(_Float16)(ov[0] * inv), (_Float16)(ov[1] * inv),
                                      (_Float16)(ov[2] * inv), (_Float16)(ov[3] * inv)};
                *reinterpret_cast<half4*>(Oh + (long long)row * D + 16 * db + 4 * g) = h;
            }
            if (g == 0) a.lse[(long long)bh * S + row] = (m_run[qb] * a.c + log2f(lt)) * kLn2;
        }
    }
}

using Shape64 = Shape<64, 2, 4, 64>;
using Shape128 = Shape<128, 2, 4, 64>;

template <class SH, bool CAUSAL>
hipError_t launch_shape(const LaunchArgs& a, hipStream_t stream) {
    KernelArgs k;
    k.q = static_cast<const _Float16*>(a.q);
    k.k = static_cast<const _Float16*>(a.k);
    k.v = static_cast<const _Float16*>(a.v);
    k.o = static_cast<_Float16*>(a.o);
    k.lse = a.lse;
    k.S = a.S;
    k.BH = a.B * a.H;
    k.nqt = (a.S + SH::BM - 1) / SH::BM;
    k.nblocks = k.BH * k.nqt;
    k.c = (float)((double)a.scale * kLog2e);
    auto kern = fa2_fwd_kernel<SH, CAUSAL>;
    if (SH::LDS_BYTES > 65536) {
        static bool attr_set = false;  // per process; the attribute is per function
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               SH::LDS_BYTES);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
    }
    hipLaunchKernelGGL(kern, dim3(k.nblocks), dim3(SH::THREADS), SH::LDS_BYTES, stream, k);
    return hipGetLastError();
}

}  // namespace

TileShape tile_shape(int D, int /*causal*/) {
    if (D == 128) return {Shape128::BM, Shape128::BN, Shape128::THREADS, Shape128::LDS_BYTES};
    return {Shape64::BM, Shape64::BN, Shape64::THREADS, Shape64::LDS_BYTES};
}

hipError_t launch_forward(const LaunchArgs& a, hipStream_t stream) {
    if (a.D == 64) return a.causal ? launch_shape<Shape64, true>(a, stream) : launch_shape<Shape64, false>(a, stream);
    return a.causal ? launch_shape<Shape128, true>(a, stream) : launch_shape<Shape128, false>(a, stream);
}

}  // namespace fa2
