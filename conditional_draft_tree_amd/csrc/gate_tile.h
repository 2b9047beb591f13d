// gate_tile.h -- the GRU gate contraction of one workgroup tile: 16 hidden
// units x RB x 16 rows x one of `ksplit` K ranges, on bf16 MFMA with binary32
// accumulation.  Shared by the stepped contraction kernel (gru.hip) and the
// fused expansion kernel (expand.hip).  Internal; not part of the C ABI.
//
// A wave's accumulators: x waves (the token embedding) add into gates
// (r, z, n) = slots 0, 1, 2; h waves (the state) into (r, z, n) = slots 0,
// 1, 3 -- slot 2 holds the candidate gate's x part and slot 3 its h part,
// which the reset gate scales.
#pragma once

#include "dt_device.h"
#include "dt_launch.h"

namespace dt {
namespace gate {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBlocks = 4;  // up to 4 x 16 rows per workgroup
// 16-row blocks a workgroup covers: fewer when the batch is small, so that
// no activation loads are spent on rows past B
inline int row_blocks(int B) { return B <= 16 ? 1 : B <= 32 ? 2 : kRowBlocks; }

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kWaves8 = 8;
constexpr int kMaxXChunks = 6;  // x chunks per wave and batch
constexpr int kMaxHChunks = 2;  // h chunks per wave and batch
// 16-byte loads per lane of an x chunk, and of an h chunk (three activation
// parts), with rb row blocks
constexpr int x_chunk_loads(int rb) { return 3 + rb; }
constexpr int h_chunk_loads(int rb) { return 3 + 3 * rb; }

// Work split.  K is cut into 32-wide chunks: nE chunks of the x part then
// nH of the h part (three bf16 parts each, so three times the MFMAs and the
// activation loads).  Each tile of 16 hidden units is covered by ksplit
// workgroups of 8 waves; in every workgroup the first WX waves take x chunks
// and the others h chunks, so that every workgroup loads about the same
// bytes (the bytes a CU loads set the contraction's time).  WX minimizes
// the larger per-wave load of the two kinds.  A wave issues every load of
// its chunks (weights and activations) before its first MFMA: one memory
// round trip.
inline int x_waves(int nE, int nH, int ksplit, int rb) {
    if (nH == 0) return kWaves8;
    if (nE == 0) return 0;
    int best = 1;
    long long best_cost = -1;
    for (int wx = 1; wx < kWaves8; ++wx) {
        const int nx = ksplit * wx, nh = ksplit * (kWaves8 - wx);
        const long long cost = max((long long)((nE + nx - 1) / nx) * x_chunk_loads(rb),
                                   (long long)((nH + nh - 1) / nh) * h_chunk_loads(rb));
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = wx;
        }
    }
    return best;
}
// [begin, end) of the chunks of wave w (0 <= w < 8) of K range ks, with wx
// x waves per workgroup
__device__ __forceinline__ void wave_chunks(int nE, int nH, int ksplit, int wx, int ks, int w, int& cb, int& ce) {
    if (w < wx) {
        const int n = ksplit * wx, i = ks * wx + w;
        cb = (int)((long long)i * nE / n);
        ce = (int)((long long)(i + 1) * nE / n);
    } else {
        const int n = ksplit * (kWaves8 - wx), i = ks * (kWaves8 - wx) + (w - wx);
        cb = nE + (int)((long long)i * nH / n);
        ce = nE + (int)((long long)(i + 1) * nH / n);
    }
}

// The accumulators of this wave (8 waves per workgroup) for tile (unit tile
// ut, row group rg, K range ks).  WM: weight source (0: W_ih / W_hh; 1:
// those, and write the packed copy; 2: the packed copy), a template parameter
// so that each variant keeps one address path and no dead store code.  RB:
// 16-row blocks per workgroup.
template <int WM, int RB>
__device__ __forceinline__ void tile_accumulate(const GruGatesArgs& a, int ut, int rg, int ks, f32x4 (&acc)[RB][4]) {
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int unit = ut * 16 + (lane & 15);
    const int kq = (lane >> 4) * 8;  // MFMA operand layout: lane l supplies row/column
                                     // l % 16 with K values 8 * (l / 16) .. + 8
    const int nE = a.E / 32, nH = a.H / 32;
    int cbeg, cend;
    wave_chunks(nE, nH, a.ksplit, a.xwaves, ks, wave, cbeg, cend);

    const bf16_t* wi = (const bf16_t*)a.W_ih + (size_t)unit * a.E;
    const bf16_t* wh = (const bf16_t*)a.W_hh + (size_t)unit * a.H;
    const size_t gi = (size_t)a.H * a.E, gh = (size_t)a.H * a.H;  // one gate's rows
    // packed weights: the 1 KB operand tile (16 units x 32 K) of unit tile ut,
    // gate g and chunk c (x chunks, then h chunks) is contiguous; lane l's
    // 16 bytes sit at l * 16 in it (see pack_index_w)
    constexpr bool wread = WM == 2, wwrite = WM == 1;
    const size_t wgate = (size_t)(nE + nH) * 512;  // one gate of one unit tile
    // per-lane base and strides (gate, chunk) of the weight loads, either layout
    const bf16_t* wpl = (const bf16_t*)a.wpack + pack_index_w(ut, 0, 0, nE + nH) + lane * 8;
    const bf16_t* wxb = wread ? wpl : wi + kq;
    const bf16_t* whb = wread ? wpl + (size_t)nE * 512 : wh + kq;
    const size_t wxg = wread ? wgate : gi, whg = wread ? wgate : gh, wcs = wread ? 512 : 32;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    // packed activations: lane l reads row l % 16 of its row block at K offset
    // 8 * (l / 16) of a chunk; a wave's read is one contiguous 1 KB block.
    // Rows past B read the last row (their sums are not stored).
    const bf16_t* xblk[RB];
    const bf16_t* hblk[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = min(rg * 64 + rb * 16 + (lane & 15), a.B - 1);
        xblk[rb] = (const bf16_t*)a.xpack + pack_index_x(r, 0, a.E) + kq;
        hblk[rb] = (const bf16_t*)a.hpack + pack_index_h(r, 0, 0, a.H) + kq;
    }
    const size_t xstep = 16 * 32;                  // one chunk of one block
    const size_t hpart = (size_t)nH * 16 * 32;     // one part of one block

#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[rb][g] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (cbeg < nE) {
        // x part: batches of up to kMaxXChunks chunks, all loads of a batch at once
        for (int cb = cbeg; cb < cend; cb += kMaxXChunks) {
            const int n = min(kMaxXChunks, cend - cb);
            bf16x8 w[kMaxXChunks][3], x[kMaxXChunks][RB];
#pragma unroll
            for (int i = 0; i < kMaxXChunks; ++i) {
                const size_t c = (size_t)(cb + min(i, n - 1));  // clamped: always in bounds
#pragma unroll
                for (int g = 0; g < 3; ++g) {  // chunks past n: zero weights (no branch, see below)
                    const bf16x8 v = load_bf16x8(wxb + g * wxg + c * wcs);
                    w[i][g] = i < n ? v : zero;
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) x[i][rb] = load_bf16x8(xblk[rb] + c * xstep);
            }
            // MFMAs for every chunk slot, unconditionally, and no scheduling
            // across this point: loads sunk next to their MFMAs would wait
            // one by one (loads complete in order)
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (wwrite) {  // the round's first contraction leaves the packed copy
#pragma unroll
                for (int i = 0; i < kMaxXChunks; ++i)
                    if (i < n)
#pragma unroll
                        for (int g = 0; g < 3; ++g)
                            *reinterpret_cast<u32x4*>((bf16_t*)wpl + g * wgate + (size_t)(cb + i) * 512) =
                                __builtin_bit_cast(u32x4, w[i][g]);
            }
#pragma unroll
            for (int i = 0; i < kMaxXChunks; ++i) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    acc[rb][0] = mfma(x[i][rb], w[i][0], acc[rb][0]);
                    acc[rb][1] = mfma(x[i][rb], w[i][1], acc[rb][1]);
                    acc[rb][2] = mfma(x[i][rb], w[i][2], acc[rb][2]);
                }
            }
        }
    } else {
        // h part (three exact bf16 parts per state element)
        for (int cb = cbeg; cb < cend; cb += kMaxHChunks) {
            const int n = min(kMaxHChunks, cend - cb);
            bf16x8 w[kMaxHChunks][3], hp[kMaxHChunks][RB][3];
#pragma unroll
            for (int i = 0; i < kMaxHChunks; ++i) {
                const size_t c = (size_t)(cb + min(i, n - 1) - nE);
#pragma unroll
                for (int g = 0; g < 3; ++g) {
                    const bf16x8 v = load_bf16x8(whb + g * whg + c * wcs);
                    w[i][g] = i < n ? v : zero;
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        hp[i][rb][q] = load_bf16x8(hblk[rb] + q * hpart + c * xstep);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (wwrite) {
#pragma unroll
                for (int i = 0; i < kMaxHChunks; ++i)
                    if (i < n)
#pragma unroll
                        for (int g = 0; g < 3; ++g)
                            *reinterpret_cast<u32x4*>((bf16_t*)wpl + g * wgate + (size_t)(cb + i) * 512) =
                                __builtin_bit_cast(u32x4, w[i][g]);
            }
#pragma unroll
            for (int i = 0; i < kMaxHChunks; ++i) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        acc[rb][0] = mfma(hp[i][rb][q], w[i][0], acc[rb][0]);
                        acc[rb][1] = mfma(hp[i][rb][q], w[i][1], acc[rb][1]);
                        acc[rb][3] = mfma(hp[i][rb][q], w[i][2], acc[rb][3]);
                    }
            }
        }
    }

}

// ---- 32-unit tiles with the activations staged in LDS -----------------------
// A workgroup of 8 waves owns 32 hidden units (unit tiles 2 ug and 2 ug + 1)
// and one kind of the contraction's K range: x (the embedding part, nE
// chunks) or h (the state part, nH chunks), share ksub of nsub equal shares
// of that kind.  Workgroups of one kind only: the consumer adds nsub partial
// sums per kind rather than one per K range of either kind.  The workgroup
// copies its share's packed activations (RB row blocks; three parts per h
// chunk) into LDS once for all its waves, so each activation byte crosses
// the memory system once per 32 units.  Wave w takes unit tile w / 4 and
// quarter w % 4 of the share's chunks: the weights of its chunks are loaded
// into registers in one batch, issued with the activation copy (one memory
// round trip), and the activation operands are read from LDS.  Accumulator
// slots 0, 1, 2 hold gates r, z, n of the kind.  The weights are the MFMA's
// first operand: output lane l holds units 4 (l / 16) .. + 3 of the unit
// tile for row l % 16 of each row block (16 contiguous bytes per row).
//
// Chunks per wave: at most t32_xbatch(RB) x chunks or t32_hbatch(RB) h
// chunks (weights in registers: fewer row blocks leave room for more);
// t32_fits() is the host's check of a configuration.
__host__ __device__ constexpr int t32_xbatch(int rb) { return rb == 4 ? 8 : 12; }
__host__ __device__ constexpr int t32_hbatch(int rb) { return rb == 4 ? 4 : 6; }
constexpr int kT32Quarters = 4;  // waves per unit tile

// [b, e) of share i of n equal shares of [0, total)
__host__ __device__ inline void share(int total, int n, int i, int& b, int& e) {
    b = (int)((long long)i * total / n);
    e = (int)((long long)(i + 1) * total / n);
}
inline bool t32_fits(int nE, int nH, int ksx, int ksh, int rb) {
    const int nx = (nE + ksx - 1) / ksx, nh = (nH + ksh - 1) / ksh;  // largest shares
    return (nx + kT32Quarters - 1) / kT32Quarters <= t32_xbatch(rb) &&
           (nh + kT32Quarters - 1) / kT32Quarters <= t32_hbatch(rb);
}
// Bytes of LDS one workgroup's staged activations take (the largest share).
inline size_t t32_act_bytes(int nE, int nH, int ksx, int ksh, int rb) {
    const int nx = (nE + ksx - 1) / ksx, nh = (nH + ksh - 1) / ksh;
    return (size_t)rb * (nx > 3 * nh ? nx : 3 * nh) * 1024;
}

// Operand-tile order: lane l of an MFMA operand read takes row m = l % 16 and
// K group g = l / 16 (8 elements at K offset 8 g) of a 1 KB block, in memory
// 16-byte vector 4 m + g of the block.  In LDS the vector (m, g) sits at
// position t32_lds_pos(m, g) = 4 m + ((g - m / 4) mod 4): copy lane p then
// takes row p / 4 and K group (p + p / 16) mod 4, so that lanes 4 i .. 4 i + 3
// read one row's 64 contiguous bytes (one cache line for four lanes, where
// the operand order would touch four lines), and the operand reads of 16
// lanes (one g, rows 0 .. 15) still fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int t32_lds_pos(int m, int g) { return 4 * m + ((g - (m >> 2)) & 3); }
// The K group copy lane p takes (of row p / 4); the vector it reads in the
// packed layout.
__device__ __forceinline__ int t32_copy_group(int p) { return ((p & 3) + (p >> 4)) & 3; }
__device__ __forceinline__ int t32_src_vector(int p) { return 4 * (p >> 2) + t32_copy_group(p); }

// A wave's place in the 32-unit tile: unit tile, quarter, and its chunks
// [cb, cb + n) of the workgroup's share [sb, sb + nsh) of its kind's chunks
// (chunks numbered within the kind).  (Wave-uniform: scalar registers.)
struct T32Wave {
    int lane, wave, u, qt, ut, kq, nE, nH, nC, sb, nsh, cb, n, cg;
};
__device__ __forceinline__ T32Wave t32_wave(const GruGatesArgs& a, int ug, int kind, int ksub, int nsub) {
    T32Wave r;
    r.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    r.lane = lane_id();
    r.u = r.wave / kT32Quarters;
    r.qt = r.wave % kT32Quarters;
    r.ut = ug * 2 + r.u;
    r.kq = (r.lane >> 4) * 8;
    r.nE = a.E / 32;
    r.nH = a.H / 32;
    r.nC = r.nE + r.nH;
    int se, qb, qe;
    share(kind ? r.nH : r.nE, nsub, ksub, r.sb, se);
    r.nsh = se - r.sb;
    share(r.nsh, kT32Quarters, r.qt, qb, qe);
    r.cb = r.sb + qb;
    r.n = qe - qb;
    r.cg = kind ? r.nE : 0;  // the kind's first chunk in the packed weights
    return r;
}

// The weights of the wave's chunks into registers: from the operand-tile copy
// (PACKED) or from W_ih / W_hh in place.  A wave-uniform base plus a fixed
// per-lane byte offset per load; fully unrolled with constant trip counts (the
// array stays in registers); past n, chunk n - 1 is loaded again (its MFMAs
// are skipped).
template <int KIND, bool PACKED, int RB>
__device__ __forceinline__ void t32_load_weights(const GruGatesArgs& a, const T32Wave& r,
                                                 bf16x8 (&w)[t32_xbatch(RB)][3]) {
    constexpr int kind = KIND, NB = KIND ? t32_hbatch(RB) : t32_xbatch(RB);
    const size_t wgate = (size_t)r.nC * 512;
    const char* wpk = (const char*)a.wpack + pack_index_w(r.ut, 0, 0, r.nC) * 2;
    const int Kk = kind ? a.H : a.E;  // row length of the kind's weight matrix
    const char* wsrc = (const char*)(kind ? a.W_hh : a.W_ih) + (size_t)r.ut * 16 * Kk * 2;
    const unsigned loff = PACKED ? (unsigned)r.lane * 16u : (unsigned)(((r.lane & 15) * Kk + r.kq) * 2);
    auto wload = [&](int i, int g) {
        const int c = r.cb + min(i, r.n - 1);
        const char* base = PACKED ? wpk + (g * wgate + (size_t)(r.cg + c) * 512) * 2
                                  : wsrc + ((size_t)g * a.H * Kk + (size_t)c * 32) * 2;
        // (each weight byte is read once per launch: non-temporal, so the
        // stream does not evict what the node workgroups keep in the L2)
        return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + loff)));
    };
    if (r.n > 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int g = 0; g < 3; ++g) w[i][g] = wload(i, g);
    }
}

// Copy the share's activations into LDS (x blocks [rb][c], or h blocks
// [rb * 3 + q][c], 1 KB each; wave w copies blocks w, w + 8, ... with
// global_load_lds_dwordx4: lane l's 16 bytes land at block + 16 l, no
// registers held; cache policy CPOL), wait for them, and contract them with
// the wave's weights.  PACK: also store the weights into the operand-tile copy
// (the call's first contraction).  ROWS (persistent launch): row i < 16 RB
// of the activations starts at element roff[i] (LDS) of the embedding table
// a.x (x part, bf16) or of the binary32 states hbase (h part, which is split
// into its three bf16 parts here), instead of the packed copies.
template <int KIND, bool PACK, int RB, int CPOL, bool ROWS = false>
__device__ __forceinline__ void t32_contract(const GruGatesArgs& a, const T32Wave& r, u32x4* sact,
                                             const bf16x8 (&w)[t32_xbatch(RB)][3], f32x4 (&acc)[RB][3],
                                             const int32_t* roff = nullptr, const float* hbase = nullptr) {
    constexpr int kind = KIND, XB = t32_xbatch(RB), HB = t32_hbatch(RB);
    const int lane = r.lane, nsh = r.nsh, sb = r.sb, cb = r.cb, n = r.n;
    const int nper = kind ? 3 * RB : RB;  // block rows (rb, or rb and part)
    const int nblk = nper * nsh;
    const u32x4* src0 = reinterpret_cast<const u32x4*>(kind ? a.hpack : a.xpack);
    const int nrow = kind ? r.nH : r.nE;  // chunks per block row in the packed layout
    const int sv = t32_src_vector(lane);
    if constexpr (ROWS && KIND == 0) {
        // lane p of a block: row p / 4 of the row block, K group
        // t32_copy_group(p) of the chunk (the copy order, see above)
        const bf16_t* xrow[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
            xrow[rr] = (const bf16_t*)a.x + (unsigned)roff[rr * 16 + (lane >> 2)] + sb * 32 + t32_copy_group(lane) * 8;
        for (int blk = r.wave; blk < nblk; blk += kWaves8) {
            int rr = 0, c = blk;
            while (c >= nsh) {
                c -= nsh;
                ++rr;
            }
            const bf16_t* src = rr == 0 ? xrow[0] : rr == 1 ? xrow[min(1, RB - 1)] : rr == 2 ? xrow[min(2, RB - 1)]
                                                                                          : xrow[RB - 1];
            __builtin_amdgcn_global_load_lds(src + c * 32, (__attribute__((address_space(3))) void*)(sact + blk * 64),
                                             16, 0, 0);
        }
    } else if constexpr (ROWS && KIND == 1) {
        // the (row block, chunk) blocks of the share: lane p reads row m = p / 4's
        // states 4 j .. 4 j + 3 and 16 + 4 j .. 16 + 4 j + 3 (j = p % 4: four
        // lanes read 64 contiguous bytes per load) and writes their three
        // parts, 8 bytes each, into the blocks (rb * 3 + q, c) at the halves j %
        // 2 of vectors (m, j / 2) and (m, 2 + j / 2)
        // (batches of kHB blocks per wave: every load of a batch is issued
        // before the first is used -- no branch between them, so that none is
        // moved down to its use; past the last block a wave repeats it,
        // writing the same values again)
        constexpr int kHB = 6;
        const int nrb = RB * nsh;
        for (int i0 = r.wave; i0 < nrb; i0 += kHB * kWaves8) {
            f32x4 v[kHB][2];
#pragma unroll
            for (int j = 0; j < kHB; ++j) {
                const int i = min(i0 + j * kWaves8, nrb - 1);
                const int rr = i / nsh, c = i - rr * nsh;
                const float* src = hbase + (unsigned)roff[rr * 16 + (lane >> 2)] + (sb + c) * 32 + (lane & 3) * 4;
                v[j][0] = *reinterpret_cast<const f32x4*>(src);
                v[j][1] = *reinterpret_cast<const f32x4*>(src + 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kHB; ++j) {
                const int i = min(i0 + j * kWaves8, nrb - 1);
                const int rr = i / nsh, c = i - rr * nsh;
                uint32_t pq[3][4] = {};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t p3[3];
                    split3_bf16(v[j][e >> 2][e & 3], p3);
#pragma unroll
                    for (int q = 0; q < 3; ++q) pq[q][e >> 1] |= p3[q] << (16 * (e & 1));
                }
                const int m = lane >> 2, jj = lane & 3;
                const int pa = t32_lds_pos(m, jj >> 1), pb = t32_lds_pos(m, 2 + (jj >> 1));
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    uint32_t* blk = reinterpret_cast<uint32_t*>(sact + ((rr * 3 + q) * nsh + c) * 64);
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<u32x2*>(blk + pa * 4 + (jj & 1) * 2) = u32x2{pq[q][0], pq[q][1]};
                    *reinterpret_cast<u32x2*>(blk + pb * 4 + (jj & 1) * 2) = u32x2{pq[q][2], pq[q][3]};
                }
            }
        }
    } else {
        for (int blk = r.wave; blk < nblk; blk += kWaves8) {
            int rr = 0, c = blk;
            while (c >= nsh) {
                c -= nsh;
                ++rr;
            }
            const u32x4* src = src0 + ((size_t)rr * nrow + sb + c) * 64 + sv;
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(sact + blk * 64), 16, 0,
                                             CPOL);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < 3; ++g) acc[rb][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (n <= 0) return;
    if constexpr (PACK) {
        const size_t wgate = (size_t)r.nC * 512;
        bf16_t* wpl = (bf16_t*)a.wpack + pack_index_w(r.ut, 0, 0, r.nC) + lane * 8;
#pragma unroll
        for (int i = 0; i < (KIND ? HB : XB); ++i)
            if (i < n)  // (uniform)
#pragma unroll
                for (int g = 0; g < 3; ++g)
                    *reinterpret_cast<u32x4*>(wpl + g * wgate + (size_t)(r.cg + cb + i) * 512) =
                        __builtin_bit_cast(u32x4, w[i][g]);
    }
    // x waves read their operand fragments from LDS one chunk ahead (two
    // buffers): the MFMAs of chunk i run while chunk i + 1's reads are in
    // flight.  h waves (three times the fragments per chunk) read a chunk's
    // fragments together, then run its MFMAs.  The scheduling barrier per
    // chunk keeps the compiler from hoisting every chunk's reads (their
    // fragments would all be held in registers).
    if constexpr (KIND == 0) {
        bf16x8 f[2][RB];
        const int lp = t32_lds_pos(lane & 15, lane >> 4);
        auto rd = [&](bf16x8 (&d)[RB], int i) {
            const int c = cb + i - sb;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) d[rb] = __builtin_bit_cast(bf16x8, sact[(rb * nsh + c) * 64 + lp]);
        };
        rd(f[0], 0);
#pragma unroll
        for (int i = 0; i < XB; ++i) {
            if (i < n) {  // (uniform)
                if (i + 1 < n) rd(f[(i + 1) & 1], i + 1);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    acc[rb][0] = mfma(w[i][0], f[i & 1][rb], acc[rb][0]);
                    acc[rb][1] = mfma(w[i][1], f[i & 1][rb], acc[rb][1]);
                    acc[rb][2] = mfma(w[i][2], f[i & 1][rb], acc[rb][2]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        const int lp = t32_lds_pos(lane & 15, lane >> 4);
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            if (i < n) {  // (uniform)
                const int c = cb + i - sb;
                bf16x8 f[RB][3];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        f[rb][q] = __builtin_bit_cast(bf16x8, sact[((rb * 3 + q) * nsh + c) * 64 + lp]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        acc[rb][0] = mfma(w[i][0], f[rb][q], acc[rb][0]);
                        acc[rb][1] = mfma(w[i][1], f[rb][q], acc[rb][1]);
                        acc[rb][2] = mfma(w[i][2], f[rb][q], acc[rb][2]);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One 32-unit tile contraction: the weights (WM 2: from the operand-tile
// copy; WM 1: in place, leaving that copy) issued with the activation copy
// (one memory round trip), then the MFMAs.
template <int WM, int RB>
__device__ __forceinline__ void tile32_lds(const GruGatesArgs& a, int ug, int kind, int ksub, int nsub, u32x4* sact,
                                           f32x4 (&acc)[RB][3]) {
    const T32Wave r = t32_wave(a, ug, kind, ksub, nsub);
    bf16x8 w[t32_xbatch(RB)][3];
    if (kind == 0) {
        t32_load_weights<0, WM == 2, RB>(a, r, w);
        t32_contract<0, WM == 1, RB, 0>(a, r, sact, w, acc);
    } else {
        t32_load_weights<1, WM == 2, RB>(a, r, w);
        t32_contract<1, WM == 1, RB, 0>(a, r, sact, w, acc);
    }
}

// The weights of a workgroup's share (both unit tiles, the four quarters)
// copied from W_ih / W_hh into the operand-tile layout of pack_index_w: the
// same chunks tile32_lds<2, RB> of that workgroup reads afterwards.
__device__ __forceinline__ void t32_pack_weights(const GruGatesArgs& a, int ug, int kind, int ksub, int nsub) {
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave), lane = lane_id();
    const int u = wave / kT32Quarters, qt = wave % kT32Quarters;
    const int ut = ug * 2 + u;
    const int nE = a.E / 32, nH = a.H / 32, nC = nE + nH;
    int sb, se, qb, qe;
    share(kind ? nH : nE, nsub, ksub, sb, se);
    share(se - sb, kT32Quarters, qt, qb, qe);
    const int cg = kind ? nE : 0, Kk = kind ? a.H : a.E;
    const bf16_t* src = (const bf16_t*)(kind ? a.W_hh : a.W_ih) + ((size_t)ut * 16 + (lane & 15)) * Kk + (lane >> 4) * 8;
    bf16_t* dst = (bf16_t*)a.wpack + pack_index_w(ut, 0, 0, nC) + lane * 8;
    const size_t wgate = (size_t)nC * 512;
    for (int c = sb + qb; c < sb + qe; ++c)
#pragma unroll
        for (int g = 0; g < 3; ++g)
            *reinterpret_cast<u32x4*>(dst + g * wgate + (size_t)(cg + c) * 512) =
                *reinterpret_cast<const u32x4*>(src + (size_t)g * a.H * Kk + (size_t)c * 32);
}

}  // namespace gate
}  // namespace dt
