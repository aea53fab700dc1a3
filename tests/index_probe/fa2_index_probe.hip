// Host-side entry points into the kernel's index arithmetic (fa2_index.h), for
// the CPU tests: they compare their numpy emulation of the mapping, the
// swizzles and the lane offsets with what the kernel itself computes. No GPU
// code and no GPU call; test infrastructure only.
#include "fa2_index.h"

using namespace fa2;

extern "C" {

// which: 0 = K swizzle, 1 = V swizzle, 2 = V swizzle of the 32x32x16 path.
int fa2_probe_swizzle(int which, int D, int row) {
    if (which == 2) return swz_v32(row);
    if (D == 64) return which == 0 ? swz_k<64>(row) : swz_v<64>(row);
    return which == 0 ? swz_k<128>(row) : swz_v<128>(row);
}

// The workgroup -> (bh, qt) mapping for every bid in [0, nblocks_grid). mask: 0
// none, 1 causal, 2 window. cu (host memory, nseq+1 entries) selects the packed
// path; its ranking (lpt) is the kernel's rule restated for one thread: the
// sequence whose count of sequences ranking before it (longer, or as long with
// a lower index), over clamped lengths, is rho. Writes bh = qt = -1 for a
// workgroup with no work.
void fa2_probe_map_blocks(int mask, int nqt, int group, int BH, int BHkv, int H, int nblocks, int serp, int lpt,
                          const int* cu, int nseq, int total, int S, int nblocks_grid, int* bh, int* qt) {
    KernelArgs a{};
    a.cu = cu;
    a.nqt = nqt;
    a.group = group;
    a.BH = BH;
    a.BHkv = BHkv;
    a.H = H;
    a.nblocks = nblocks;
    a.serp = serp;
    a.lpt = lpt;
    a.total = total;
    a.S = S;
    auto rank_of = [&](int n, int rho) {
        auto len = [&](int j) {
            int s0 = cu[j] < 0 ? 0 : (cu[j] > total ? total : cu[j]);
            int s1 = cu[j + 1] < s0 ? s0 : (cu[j + 1] > total ? total : cu[j + 1]);
            return (s1 - s0) < S ? (s1 - s0) : S;
        };
        for (int j = 0; j < n; ++j) {
            int rank = 0;
            for (int i = 0; i < n; ++i) rank += (len(i) > len(j)) || (len(i) == len(j) && i < j);
            if (rank == rho) return j;
        }
        return 0;
    };
    (void)nseq;
    for (int bid = 0; bid < nblocks_grid; ++bid) {
        int b = -1, q = -1;
        bool ok = mask == 1 ? map_block<kCausal>(a, bid, b, q, rank_of)
                : mask == 2 ? map_block<kWindow>(a, bid, b, q, rank_of)
                            : map_block<kNoMask>(a, bid, b, q, rank_of);
        bh[bid] = ok ? b : -1;
        qt[bid] = ok ? q : -1;
    }
}

// Per-lane K/V load offsets for the tile shapes the kernel instantiates
// (D 64 or 128, NW 4 or 8; mf32 only at D = 64).
int fa2_probe_lane_load_offsets(int D, int NW, int mf32, int kv_sr, int wave, int lane, int* row0,
                                uint32_t* offK, uint32_t* offV) {
    if (D == 64 && NW == 8 && !mf32) lane_load_offsets<64, 8, false>(wave, lane, kv_sr, *row0, *offK, *offV);
    else if (D == 64 && NW == 4 && !mf32) lane_load_offsets<64, 4, false>(wave, lane, kv_sr, *row0, *offK, *offV);
    else if (D == 64 && NW == 8 && mf32) lane_load_offsets<64, 8, true>(wave, lane, kv_sr, *row0, *offK, *offV);
    else if (D == 64 && NW == 4 && mf32) lane_load_offsets<64, 4, true>(wave, lane, kv_sr, *row0, *offK, *offV);
    else if (D == 128 && NW == 8 && !mf32) lane_load_offsets<128, 8, false>(wave, lane, kv_sr, *row0, *offK, *offV);
    else if (D == 128 && NW == 4 && !mf32) lane_load_offsets<128, 4, false>(wave, lane, kv_sr, *row0, *offK, *offV);
    else return -1;
    return 0;
}

int fa2_probe_lds_read_bases(int D, int lane, uint32_t* rdK0, uint32_t* rdV0) {
    if (D == 64) lds_read_bases<64>(lane, *rdK0, *rdV0);
    else if (D == 128) lds_read_bases<128>(lane, *rdK0, *rdV0);
    else return -1;
    return 0;
}

}  // extern "C"
