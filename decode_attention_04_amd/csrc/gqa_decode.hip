// Single-token GQA flash-decode attention over a bf16 KV cache, gfx950 only.
//
// The split-KV scheme of the AstrAI csrc commit log (split-KV bullets) with the
// partial/fold structure of sparkinfer PR #877 (section Mechanism):
//
//   gqa_split_kernel   a workgroup of four waves takes a key range of one
//                      (sequence b, kv head) segment -- a fixed split, or a
//                      piece of an even share of the concatenated tiles of all
//                      segments -- for all G query heads of the kv head, and
//                      emits one unnormalised partial (m, l, acc) per query
//                      head, or the output itself when its range is the whole
//                      segment.
//   gqa_combine_kernel / gqa_combine_narrow_kernel
//                      fold the partials of each (b, h) with the log-sum-exp
//                      rescale in a fixed order (a tree for many partials, one
//                      thread per column for few).
//   With the in-kernel fold (the default where a segment's fixed splits make
//   one small fold, a tuning choice elsewhere), the split workgroup that writes
//   the last partial of a group (an arrival ticket tells it) folds the group
//   itself and the combine kernel is not launched.
//
// The default pipeline inside one wave (64 lanes, r = lane % 16, grp = lane / 16):
//
//   K/V   16-byte raw buffer loads with the non-temporal hint; the buffer
//         bounds end at the sequence length, so rows past it read as zero and
//         a NaN in an unused cache tail never reaches a sum.  One register tile
//         per wave (16 keys at head_dim >= 128), refilled part by part as soon
//         as each part is dead, so the next tile's loads fly during this
//         tile's math (the role of the shared-memory double buffer of
//         sparkinfer PR #874, section Summary).
//   QK^T  v_mfma_f32_16x16x32_bf16 with A = 16 keys x 32 dims straight from the
//         load registers and B = 32 dims x 16 query rows (the G heads of the kv
//         head, zero padded); Q is exact bf16, resident in the B operand.  Lane
//         (r, grp) receives the scores of query row r for keys 4*grp .. +3.
//   softmax  the scale (times log2 e) applied to the fp32 scores; the running
//         max of row r is shared by lanes r, r+16, r+32, r+48 through the
//         gfx950 lane swaps; l is kept per lane and summed once at the end.
//   PV    bf16 MFMAs with P split into bf16 hi + lo parts (P = hi + lo to about
//         2^-17 relative); V staged row-major in a per-wave LDS buffer and read
//         back by transposing LDS reads; the accumulator's column is the lane's
//         own query row, so the softmax rescale is lane-local.
//   Ranges of at most four tiles (one per wave) run in lock step instead: two
//   LDS exchanges (row maxima, then the probabilities against the range's
//   maximum) and PV split by head-dim quarters, with no fold afterwards.
//
// A/B variants kept for same-binary comparison (gqa_tuning_t): PV on fp32
// MFMAs (v_mfma_f32_16x16x4_f32 on V widened from the load registers), two
// register tiles per wave, QK^T on the vector ALU, the default cache policy,
// the tree combine for every plan, the in-kernel fold everywhere.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <tuple>
#include <unordered_map>
#include <utility>

#include "gqa_decode.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;           // waves per workgroup
constexpr int kPartitionFixed = 0;  // see "work partition" below
constexpr int kPartitionEven = 1;
// Proportional splits (a plan partition): run by the even-partition kernels
// with SplitArgs::prop / CombineArgs::prop set.
constexpr int kPartitionProp = 2;
constexpr int kMaxHeadsPerKv = 16;  // G is padded to the MFMA's 16 columns
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords (gfx9 family)

// Partials are blocks of [G][D] (acc) and [G][2] (m in log2 units, l), one
// per slot (see "work partition" below for the slot numbering).
struct SplitArgs {
    const uint16_t *q;
    const unsigned char *k;     // bf16 or E4M3 cache, addressed in bytes
    const unsigned char *v;
    const int32_t *seq_lens;
    const int32_t *page_table;  // paged only
    float *part_acc;
    float *part_ml;
    float *out;                 // [B][Hq][D]
    int B, Hq, Hkv, G;          // G: query heads per kv head
    int M, R;                   // query tokens per sequence (the last M positions); R = M * G rows
    int qdiv;                   // ceil(256 / G): row r belongs to query token (r * qdiv) >> 8
    int S_max;                  // contiguous capacity
    int page_size, max_pages;   // paged
    int page_shift;             // paged: log2(page_size) when a power of two, else -1
    int num_pages;              // paged
    int num_splits, split_tokens;
    int piece_cost;             // even partition: tiles a piece's start and fold are worth
    int halve_long;             // even partition, contiguous cache: one share per CU for long segments
    float qk_scale_log2;        // scale * log2(e) (times k_scale for an E4M3 cache)
    float v_scale;              // E4M3 cache: V's per-tensor scale
    unsigned *counters;         // in-kernel fold: the arrival counters (workspace header)
    int fused;                  // 1: this kernel folds the partials itself
    int fanin;                  // fused fixed splits: partials per node of the fold tree
    int prop;                   // even-partition kernel: proportional splits instead of shares
};

struct CombineArgs {
    const float *part_acc;
    const float *part_ml;
    float *out;
    const int32_t *seq_lens;  // even partition only
    int D, G, Hq, num_splits; // G, Hq: output rows per (sequence, kv head) and per sequence
    int B, Hkv, cap, tile;    // even partition: how the split kernel cut the tiles
    int shares;               // even partition: workgroups of the split kernel
    int M, Gh;                // query tokens per sequence, query heads per kv head (G = M * Gh)
    int piece_cost;           // even partition: as in SplitArgs
    int halve_long;           // as in SplitArgs
    int prop;                 // proportional splits (thread-per-column combine only)
};

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// Cross-row exchanges (gfx950 VALU lane swaps, no LDS round trip).
// rows16: for a lane in rows (2k, 2k+1) of 16 lanes, x in row 2k and in row
// 2k+1 at the same position; halves32: x in the lower and the upper half of
// the wave at the same position.  Both lanes of a pair get the same two values.
struct LanePair {
    float lo, hi;
};
__device__ __forceinline__ LanePair rows16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(p[0]), __uint_as_float(p[1])};
}
__device__ __forceinline__ LanePair halves32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(p[0]), __uint_as_float(p[1])};
}
// Max and sum over the four lanes r, r+16, r+32, r+48 (the result in all four).
__device__ __forceinline__ float max_rows(float x) {
    LanePair p = rows16(x);
    p = halves32(fmaxf(p.lo, p.hi));
    return fmaxf(p.lo, p.hi);
}
__device__ __forceinline__ float sum_rows(float x) {
    LanePair p = rows16(x);
    p = halves32(p.lo + p.hi);
    return p.lo + p.hi;
}
// x of lane (i - n) mod 16 in this lane's row of 16.
__device__ __forceinline__ float row_ror(float x, int n) {
    switch (n) {
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
        case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
        case 8: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
        default: return x;
    }
}

template <int D>
struct Shape {
    static constexpr int KB = D / 32;                  // 32-dim blocks of the QK contraction
    static constexpr int DPL = D >= 128 ? 8 : D / 16;  // V values per lane per chunk
    static constexpr int VC = D / (16 * DPL);          // V chunks per key per lane
    static constexpr int NACC = D / 16;                // PV accumulators (f32x4) per lane
    static constexpr int VW = DPL / 2;                 // dwords per V chunk
};

// Element type of the KV cache: bf16, or OCP FP8 E4M3 with per-tensor scales
// (dequantised exactly to bf16 in registers: every E4M3 value is a bf16 value).
constexpr int kKvBf16 = 0;
constexpr int kKvFp8 = 1;

// Head dims that contraction slot (k-block kb, lane group grp) of QK^T covers:
// 8 consecutive dims starting at kslot_lane(grp) + kslot_block(kb).  The
// contraction order is free as long as K and Q agree; for E4M3 each lane loads
// 16 consecutive bytes that feed two k-blocks.
template <int KV>
__device__ __forceinline__ constexpr int kslot_lane(int grp) {
    return KV == kKvFp8 ? 16 * grp : 8 * grp;
}
template <int KV>
__device__ __forceinline__ constexpr int kslot_block(int kb) {
    return KV == kKvFp8 ? 64 * (kb >> 1) + 8 * (kb & 1) : 32 * kb;
}

// One wave's tile as loaded: NB blocks of 16 keys.
//   k[blk][w]: key 16*blk + r; bf16: k-block w, dims kslot_lane(grp) + kslot_block(w) ..;
//              E4M3: 16 bytes for k-blocks 2w and 2w + 1.
//   v[blk][j][c]: key 16*blk + 4*grp + j, dims 16*DPL*c + DPL*r .. (DPL values).
template <int D, int NB, int KV>
struct Tile {
    static constexpr int KW = KV == kKvFp8 ? Shape<D>::KB / 2 : Shape<D>::KB;  // 16-byte K loads
    static constexpr int VWL = KV == kKvFp8 ? Shape<D>::VW / 2 : Shape<D>::VW; // V dwords as loaded
    u32x4_t k[NB][KW];
    unsigned int v[NB][4][Shape<D>::VC][VWL];
};

// 4 E4M3 bytes -> 4 bf16 values (exact), packed in two dwords in byte order.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16(unsigned int w) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2_t{__builtin_bit_cast(unsigned int, lo), __builtin_bit_cast(unsigned int, hi)};
}

// The QK^T A operand of k-block kb for block blk of the tile, as bf16.
template <int D, int NB, int KV>
__device__ __forceinline__ bf16x8_t k_operand(const Tile<D, NB, KV> &t, int blk, int kb) {
    if constexpr (KV == kKvFp8) {
        const u32x4_t raw = t.k[blk][kb >> 1];
        const u32x2_t a = e4m3x4_to_bf16((kb & 1) ? raw[2] : raw[0]);
        const u32x2_t b = e4m3x4_to_bf16((kb & 1) ? raw[3] : raw[1]);
        return __builtin_bit_cast(bf16x8_t, u32x4_t{a[0], a[1], b[0], b[1]});
    } else {
        return __builtin_bit_cast(bf16x8_t, t.k[blk][kb]);
    }
}

// Dword w (of VW) of V chunk (blk, j, c) as bf16 pairs.
template <int D, int NB, int KV>
__device__ __forceinline__ unsigned int v_word(const Tile<D, NB, KV> &t, int blk, int j, int c, int w) {
    if constexpr (KV == kKvFp8) {
        return e4m3x4_to_bf16(t.v[blk][j][c][w >> 1])[w & 1];
    } else {
        return t.v[blk][j][c][w];
    }
}

// Issue the loads of one tile.  `rk` / `rv` cover the rows of this tile's
// (sequence, kv head) or page, ending at the last valid row; `row0` is the
// tile's first row inside that range.
constexpr int kLoadK = 1;
constexpr int kLoadV = 2;

// Cache policy of the K/V loads: 0 = default, kNonTemporal = the "nt" bit
// (streamed data that is not re-read; on gfx950 it lets large caches stream
// at a markedly higher rate).
constexpr int kNonTemporal = 2;
// Cache policy of the partial stores: the "sc1" (device scope) bit.
constexpr int kDeviceScope = 16;

template <int D, int NB, int CPOL, int KV>
__device__ __forceinline__ void load_tile(Tile<D, NB, KV> &t, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, int row0, int r, int grp,
                                          int parts) {
    using S = Shape<D>;
    using T = Tile<D, NB, KV>;
    constexpr int EB = KV == kKvFp8 ? 1 : 2;  // bytes per element
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        const int krow = row0 + 16 * blk + r;
#pragma unroll
        for (int w = 0; w < T::KW && (parts & kLoadK); ++w) {
            const int off = KV == kKvFp8 ? krow * D + 64 * w + 16 * grp
                                         : (krow * D + kslot_lane<KV>(grp) + kslot_block<KV>(w)) * 2;
            t.k[blk][w] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, CPOL));
        }
#pragma unroll
        for (int j = 0; j < 4 && (parts & kLoadV); ++j) {
            const int vrow = row0 + 16 * blk + 4 * grp + j;
#pragma unroll
            for (int c = 0; c < S::VC; ++c) {
                const int off = (vrow * D + 16 * S::DPL * c + S::DPL * r) * EB;
                if constexpr (T::VWL == 4) {
                    u32x4_t x = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, CPOL));
                    t.v[blk][j][c][0] = x[0];
                    t.v[blk][j][c][1] = x[1];
                    t.v[blk][j][c][2] = x[2];
                    t.v[blk][j][c][3] = x[3];
                } else if constexpr (T::VWL == 2) {
                    u32x2_t x = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, CPOL));
                    t.v[blk][j][c][0] = x[0];
                    t.v[blk][j][c][1] = x[1];
                } else {
                    t.v[blk][j][c][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, CPOL);
                }
            }
        }
    }
}

// How PV is computed:
//   kPvF32  v_mfma_f32_16x16x4_f32 on V widened to fp32 straight from the
//           load registers (exact products, 2048 MFMA cycles per 16 keys at
//           head_dim 256);
//   kPvBf16 bf16 MFMAs with P split into bf16 hi + lo parts (P = hi + lo to
//           about 2^-17 relative) and V transposed through a per-wave LDS
//           buffer (8x fewer MFMA cycles than kPvF32): v_mfma_f32_16x16x16_bf16
//           per 16 keys in key ranges; in one-tile ranges 32-deep MFMAs over
//           pairs of 16-key blocks (process_single).
constexpr int kPvF32 = 0;
constexpr int kPvBf16 = 1;

// Running online-softmax state of one wave (lane (r, grp) holds query head r).
//   kPvF32:  acc[c*DPL + e][i] = O[r][16*DPL*c + DPL*(4*grp+i) + e]
//   kPvBf16: acc[nb][i]        = O[r][16*nb + 4*grp + i]
template <int D>
struct WaveState {
    f32x4_t acc[Shape<D>::NACC];
    float m;                      // running max (log2 units), identical in the 4 lanes of head r
    float l;                      // this lane's share of the running sum
};

// Row stride (in bf16) of a wave's V staging buffer.  The padding puts the
// four key rows that a transposing read gathers per lane group on distinct
// LDS banks (rows 32 bytes apart modulo 256 for D >= 128, 144 for D = 64)
// and keeps rows aligned for the stores (16 bytes for D >= 128, 8 for D = 64,
// which also keeps the largest D = 64 tile within four workgroups per CU).
template <int D>
constexpr int kStageStride = D == 64 ? D + 8 : D + 16;

// kPvBf16: V rows of a tile (as loaded: key 16*blk + 4*grp + j, dims
// 16*DPL*c + DPL*r ..) into the wave's LDS staging buffer.
template <int D, int NB, int KV>
__device__ __forceinline__ void stage_v(const Tile<D, NB, KV> &t, int r, int grp, unsigned short *stage) {
    using S = Shape<D>;
    constexpr int RS = kStageStride<D>;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < S::VC; ++c) {
                unsigned short *dst = stage + (16 * blk + 4 * grp + j) * RS + 16 * S::DPL * c + S::DPL * r;
                if constexpr (S::VW == 4) {
                    *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{v_word(t, blk, j, c, 0), v_word(t, blk, j, c, 1),
                                                                v_word(t, blk, j, c, 2), v_word(t, blk, j, c, 3)};
                } else if constexpr (S::VW == 1) {  // head_dim 32
                    *reinterpret_cast<unsigned int *>(dst) = v_word(t, blk, j, c, 0);
                } else {
                    *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{v_word(t, blk, j, c, 0), v_word(t, blk, j, c, 1)};
                }
            }
}

// Zero the V rows of a tile at or past key `len` (the tile's first key is t0):
// a tile loaded against the cache capacity instead of the length holds
// whatever lies beyond the sequence there, and p = 0 must meet a finite V.
template <int D, int NB, int KV>
__device__ __forceinline__ void zero_v_past(Tile<D, NB, KV> &t, int t0, int len, int grp) {
    using T = Tile<D, NB, KV>;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool keep = t0 + 16 * blk + 4 * grp + j < len;
#pragma unroll
            for (int c = 0; c < Shape<D>::VC; ++c)
#pragma unroll
                for (int w = 0; w < T::VWL; ++w) t.v[blk][j][c][w] = keep ? t.v[blk][j][c][w] : 0u;
        }
}

// How QK^T is computed:
//   kQkMfma  v_mfma_f32_16x16x32_bf16 with K as the A operand straight from the
//            load registers and Q resident as the B operand (the default);
//   kQkValu  the same K registers on the vector ALU: each lane owns a quarter
//            of the head dims of one key (the A-operand layout), forms its
//            partial dot product with every query row by v_dot2c_f32_bf16
//            against a per-wave LDS copy of Q, the four quarters of a key are
//            summed by two lane swaps, and a per-wave LDS transpose hands
//            each lane the MFMA result layout.  An A/B variant (bf16 cache,
//            bf16 PV, one register tile, head_dim 128 or 256).
constexpr int kQkMfma = 0;
constexpr int kQkValu = 1;

template <int D, bool VALU>
struct QkLds {};
template <int D>
struct QkLds<D, true> {
    // 16-byte aligned: both are read and written 16 bytes per lane
    alignas(16) unsigned q[kWaves][kMaxHeadsPerKv][D / 2];  // each wave's copy of its Q rows, bf16 pairs
    alignas(16) float x[kWaves][kMaxHeadsPerKv][20];        // each wave's score transpose (rows of 80 bytes)
};

// A dword as two bf16 values.  (Taken through a scalar parameter: a bit cast
// of an element of a vector value, __builtin_bit_cast(T, v[j]), compiled to
// element 0 for every j with hipcc of ROCm 7.2.)
__device__ __forceinline__ bf16x2_t as_bf16x2(unsigned w) { return __builtin_bit_cast(bf16x2_t, w); }

// Orders a wave's own LDS writes before its following LDS reads by other lanes
// (a wave's LDS instructions execute in program order; this keeps the
// compiler from reordering them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// kQkValu: this wave's Q rows (from the B-operand registers) into its LDS copy.
template <int D>
__device__ __forceinline__ void stage_q_valu(const bf16x8_t (&qb)[Shape<D>::KB], unsigned *qtab, int r, int grp) {
#pragma unroll
    for (int kb = 0; kb < Shape<D>::KB; ++kb)
        *reinterpret_cast<u32x4_t *>(qtab + r * (D / 2) + 4 * grp + 16 * kb) = __builtin_bit_cast(u32x4_t, qb[kb]);
    wave_lds_sync();
}

// QK^T of block blk (16 keys) of a tile: lane (r, grp) gets the scores of
// query row r for keys 4*grp .. 4*grp + 3 of the block (rows >= R: zero).
template <int D, int NB, int KV, int QKM>
__device__ __forceinline__ f32x4_t qk_block(const Tile<D, NB, KV> &t, int blk, const bf16x8_t (&qb)[Shape<D>::KB],
                                            const unsigned *qtab, float *xs, int r, int grp, int R) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
    if constexpr (QKM == kQkMfma) {
#pragma unroll
        for (int kb = 0; kb < Shape<D>::KB; ++kb)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(t, blk, kb), qb[kb], c, 0, 0, 0);
    } else {
        static_assert(KV == kKvBf16, "the VALU QK^T variant reads bf16 K registers");
        float part[kMaxHeadsPerKv];
#pragma unroll
        for (int h = 0; h < kMaxHeadsPerKv; ++h) {
            part[h] = 0.f;
            if (h < R) {
                float acc = 0.f;
#pragma unroll
                for (int kb = 0; kb < Shape<D>::KB; ++kb) {
                    const u32x4_t qv = *reinterpret_cast<const u32x4_t *>(qtab + h * (D / 2) + 4 * grp + 16 * kb);
                    const u32x4_t kw = t.k[blk][kb];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[j]), as_bf16x2(qv[j]), acc, false);
                }
                part[h] = sum_rows(acc);  // key r, all its head dims (in the four lanes of key r)
            }
        }
        if (grp == 0) {
#pragma unroll
            for (int h = 0; h < kMaxHeadsPerKv; ++h) xs[h * 20 + r] = part[h];
        }
        wave_lds_sync();
        c = *reinterpret_cast<const f32x4_t *>(xs + r * 20 + 4 * grp);
        wave_lds_sync();  // read before the next block's writes
    }
    return c;
}

// QK^T and the online-softmax update for one tile whose first key has index
// `t0` in the sequence (keys at or beyond `t_end`, this lane's row limit,
// masked).  On return
// sc[blk][i] holds the probability of key 16*blk + 4*grp + i for head r
// (relative to the new running max) and acc has been rescaled.
template <int D, int NB, int KV, int QKM = kQkMfma>
__device__ __forceinline__ void qk_softmax(const Tile<D, NB, KV> &t, const bf16x8_t (&qb)[Shape<D>::KB],
                                           WaveState<D> &st, int t0, int t_end, int grp,
                                           float qk_scale_log2, f32x4_t (&sc)[NB], const unsigned *qtab = nullptr,
                                           float *xs = nullptr, int r = 0, int R = 0) {
    using S = Shape<D>;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) sc[blk] = qk_block<D, NB, KV, QKM>(t, blk, qb, qtab, xs, r, grp, R);
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * blk + 4 * grp + i;
            const float x = tok < t_end ? sc[blk][i] * qk_scale_log2 : -INFINITY;
            sc[blk][i] = x;
            mx = fmaxf(mx, x);
        }
    }
    mx = max_rows(mx);
    const float m_new = fmaxf(st.m, mx);
    // m_new is -inf only while every key this row has seen is masked (a
    // multi-query row whose causal limit lies before the tile): exponentials
    // are then taken against 0, every p is 0 and the state stays empty.
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_ref);  // 0 on the first tile
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[blk][i] - m_ref);
            sc[blk][i] = p;
            psum += p;
        }
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int a = 0; a < S::NACC; ++a) st.acc[a] *= alpha;
}

// PV for one tile with probabilities sc (see qk_softmax).
template <int D, int NB, int PV, int KV>
__device__ __forceinline__ void pv_tile(const Tile<D, NB, KV> &t, const f32x4_t (&sc)[NB], WaveState<D> &st,
                                        int r, int grp, const unsigned short *stage) {
    using S = Shape<D>;
    constexpr int RS = kStageStride<D>;
    if constexpr (PV == kPvF32) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p = sc[blk][j];
#pragma unroll
                for (int c = 0; c < S::VC; ++c) {
#pragma unroll
                    for (int e = 0; e < S::DPL; ++e) {
                        const float vf = (e & 1) ? bf16_hi(v_word(t, blk, j, c, e >> 1)) : bf16_lo(v_word(t, blk, j, c, e >> 1));
                        st.acc[c * S::DPL + e] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(vf, p, st.acc[c * S::DPL + e], 0, 0, 0);
                    }
                }
            }
        }
    } else {
        // O^T[d][g] += V^T[d][t] P^T[t][g] over the 16 keys of each block: the B
        // operand is the lane's own four probabilities (keys 4*grp + i), the A
        // operand the four V values V[4*grp + i][16*nb + r], gathered from the
        // row-major staging buffer by one transposing LDS read: within each
        // group of 16 lanes, lane r receives element r % 4 of the 8-byte row
        // pieces that lanes 4*i + r / 4 point at, so lane r points at key
        // 4*grp + r / 4, dims 16*nb + 4*(r % 4) .. + 3.
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            bf16x4_t hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hi[i] = (__bf16)sc[blk][i];
                lo[i] = (__bf16)(sc[blk][i] - (float)hi[i]);
            }
            const unsigned short *src = stage + (16 * blk + 4 * grp + (r >> 2)) * RS + 4 * (r & 3);
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const bf16x4_t av = __builtin_bit_cast(
                    bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(src + 16 * nb)));
                st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, hi, st.acc[nb], 0, 0, 0);
                st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, lo, st.acc[nb], 0, 0, 0);
            }
        }
    }
}

// QK^T, online softmax and PV for one staged tile.
template <int D, int NB, int PV, int KV>
__device__ __forceinline__ void compute_tile(const Tile<D, NB, KV> &t, const bf16x8_t (&qb)[Shape<D>::KB],
                                             WaveState<D> &st, int t0, int t_end, int r, int grp,
                                             float qk_scale_log2, unsigned short *stage) {
    if constexpr (PV == kPvBf16) stage_v(t, r, grp, stage);
    f32x4_t sc[NB];
    qk_softmax(t, qb, st, t0, t_end, grp, qk_scale_log2, sc);
    pv_tile<D, NB, PV>(t, sc, st, r, grp, stage);
}

// Per-wave LDS region: the V staging buffer during the tile loop, then the
// wave's accumulator rows [16][D + 4] fp32 for the fold (+4 floats so that
// consecutive rows start on other banks).  Each wave only ever touches its
// own region until the workgroup barrier, so the two uses never overlap.
template <int D, int NB, int QKM = kQkMfma>
struct FoldLds {
    static constexpr int kFoldBytes = kMaxHeadsPerKv * (D + 4) * 4;
    static constexpr int kStageBytes = 16 * NB * kStageStride<D> * 2;
    static constexpr int kRegion = kFoldBytes > kStageBytes ? kFoldBytes : kStageBytes;
    float m[kWaves][kMaxHeadsPerKv];
    float l[kWaves][kMaxHeadsPerKv];
    alignas(16) unsigned char region[kWaves][kRegion];
    u32x4_t p[kWaves][NB][64];  // one-tile ranges: each wave's probabilities (bf16 hi, lo), in its lane layout
    unsigned ticket[2];         // in-kernel fold: arrival tickets
    QkLds<D, QKM == kQkValu> qk;
    __device__ float *acc(int w) { return reinterpret_cast<float *>(region[w]); }
    __device__ unsigned short *stage(int w) { return reinterpret_cast<unsigned short *>(region[w]); }
};

// Minimum waves per SIMD the compiler must leave room for (256 VGPRs each at
// two): the plans launch at most two workgroups of four waves per CU in the
// even partition and one per CU for a single sequence, and both key-range
// paths of a kernel must fit without spills at every head_dim and tile.
template <int D, int NB, bool DBUF>
constexpr int kMinWavesPerEu = DBUF ? 1 : 2;

// ------------------------------------------------------------ work partition
//
// The keys of one (sequence b, kv head) pair form a "segment" of
// n_b = ceil(len_b / tile) tiles; segments are ordered b-major, kv-head-minor
// (segment index i = b*Hkv + kvh).  Two partitions of the segments onto
// workgroups exist:
//   fixed  every segment is cut into S splits of split_tokens keys; workgroup
//          (b, kvh, s) takes split s (the AstrAI split-KV scheme).  Partial slot
//          of a split: (b*Hkv + kvh)*S + s.
//   even   the concatenated tiles of all segments are cut into P equal shares,
//          share w = tiles [floor(w*N/P), floor((w+1)*N/P)) of the N tiles,
//          computed on the device from seq_lens, so a ragged batch gives every
//          workgroup the same work (the length-aware scheduling that the pages'
//          split rule leaves open).  A share may cover the end of one segment
//          and the start of the next: each such piece is folded on its own and
//          written to partial slot w + i (unique: along the tile axis every new
//          piece starts a new share, a new segment or both, so w + i grows).

__device__ __forceinline__ int clamp_len(const int32_t *seq_lens, int b, int cap) {
    return min(max(seq_lens[b], 0), cap);
}

// seq_lens[b] through the vector memory path (a buffer load), so that the
// wave can issue it before the scalar kernel-argument fetches complete and
// wait for the two independently.
__device__ __forceinline__ int load_len_vmem(const int32_t *seq_lens, int b) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)seq_lens, (short)0, (b + 1) * 4, kRsrcWord3);
    return __builtin_amdgcn_raw_buffer_load_b32(r, b * 4, 0, 0);
}

// seq_lens[b] for a b that may be B (no such sequence: 0), through the buffer bounds.
__device__ __forceinline__ int load_len_or_zero(const int32_t *seq_lens, int b, int B) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)seq_lens, (short)0, B * 4, kRsrcWord3);
    return __builtin_amdgcn_raw_buffer_load_b32(r, b * 4, 0, 0);
}

// page_table[b][i] for a b that may be B and an i that may be past max_pages (0 then).
__device__ __forceinline__ int load_page_or_zero(const int32_t *page_table, int b, int i, int B, int max_pages) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(page_table + (size_t)b * max_pages), (short)0, b < B ? max_pages * 4 : 0, kRsrcWord3);
    return __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0);
}

// Sum over the wave of an int (every lane gets the result).
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ long long uniform64(long long x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(x & 0xffffffffll));
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// A segment of n tiles spans n + K positions of the tile axis that even shares
// cut (none when n = 0): K stands for what starting and folding a piece costs,
// so that a share covering several short segments takes fewer tiles.
__device__ __forceinline__ int seg_span(int n, int K) { return n > 0 ? n + K : 0; }

// Positions of the sequences on that axis: the total of all segments, and
// (for a target position `x` < total) the sequence b whose segments hold it
// and the positions before that sequence's first segment.  Every lane of the
// wave returns the same values.
struct SegmentLocation {
    long long total;   // N: positions of all segments
    int b;             // sequence holding position x
    int len;           // its (clamped) length
    long long before;  // positions of all segments of sequences < b
};

__device__ __forceinline__ SegmentLocation locate_tile(const int32_t *seq_lens, int B, int Hkv, int cap,
                                                       int TT, int K, long long x, int lane) {
    SegmentLocation loc{0, -1, 0, 0};
    long long run = 0;  // tiles of sequences before this chunk
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int ln = bb < B ? clamp_len(seq_lens, bb, cap) : 0;
        const int n = seg_span((ln + TT - 1) / TT, K);
        const int incl = wave_scan(n, lane);
        const long long lo = (run + incl - n) * Hkv, hi = (run + incl) * Hkv;
        const unsigned long long hit = __ballot(bb < B && lo <= x && x < hi);
        if (loc.b < 0 && hit != 0ull) {
            const int l = __builtin_ctzll(hit);
            loc.b = c0 + l;
            loc.len = __shfl(ln, l, 64);
            loc.before = (run + __shfl(incl - n, l, 64)) * Hkv;
        }
        run += __shfl(incl, 63, 64);
    }
    loc.total = run * Hkv;
    // identical in every lane: keep them in scalar registers
    loc.b = __builtin_amdgcn_readfirstlane(loc.b);
    loc.len = __builtin_amdgcn_readfirstlane(loc.len);
    loc.total = uniform64(loc.total);
    loc.before = uniform64(loc.before);
    return loc;
}

// Axis positions of all segments before sequence b's first one, and of all
// segments; and the number of non-empty segments.
__device__ __forceinline__ void prefix_tiles(const int32_t *seq_lens, int B, int Hkv, int cap, int TT, int K, int b,
                                             int lane, long long &before, long long &total, long long &segs) {
    long long run = 0, pre = 0, ne = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int n = bb < B ? seg_span((clamp_len(seq_lens, bb, cap) + TT - 1) / TT, K) : 0;
        const int cnt = wave_sum(bb < b ? n : 0);
        pre += cnt;
        run += wave_sum(n);
        ne += wave_sum(n > 0 ? 1 : 0);
    }
    before = uniform64(pre * Hkv);
    total = uniform64(run * Hkv);
    segs = uniform64(ne * Hkv);
}

// Segments of a contiguous cache averaging at least this many tiles stream
// best with one share per CU: half the launched shares (the plan launches two
// per CU) then take the axis, and the other half exit at once.  Shorter
// segments, and every paged cache, keep two per CU, whose second workgroup
// covers the first one's piece starts (measured: uniform 16k-key batch 84.4 ->
// 81.8 us per call; ragged batches of up to 2k keys 48.8 -> 52.8 with one per CU).
constexpr int kLongSegmentTiles = 128;

// The number of shares the axis is cut into: the launched P, or half of it
// (halve_long, for long segments); N = axis positions, segs = non-empty segments.
__device__ __forceinline__ long long shares_for(long long P, long long N, long long segs, int K, int halve_long) {
    return (halve_long && segs > 0 && N >= (long long)(kLongSegmentTiles + K) * segs) ? (P + 1) / 2 : P;
}

// Non-empty (sequence, kv head) segments.
__device__ __forceinline__ long long nonempty_segments(const int32_t *seq_lens, int B, int Hkv, int cap, int lane) {
    long long cnt = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        cnt += wave_sum(bb < B && clamp_len(seq_lens, bb, cap) > 0 ? 1 : 0);
    }
    return uniform64(cnt * Hkv);
}

// The share of workgroup w: [share_begin(w), share_begin(w + 1)).
__device__ __forceinline__ long long share_begin(long long w, long long N, long long P) { return w * N / P; }

// Largest workgroup whose share starts at or before tile x (the one holding x).
__device__ __forceinline__ long long share_of(long long x, long long N, long long P) {
    return ((x + 1) * P + N - 1) / N - 1;
}

// Proportional splits: with N tiles in all segments and P workgroups (halved,
// as for even shares, when contiguous segments are long), every workgroup
// takes at most L = ceil(N / P) tiles: a segment of n tiles gets
// k = ceil(n / L) splits of n / k tiles (rounded down at each split start), so
// each workgroup holds exactly one piece.  Workgroups are numbered segment by
// segment in (sequence, kv head) order; the ones past the last split exit.
// Every lane of the wave returns the same values.
struct PropTotals {
    long long N;  // tiles of all segments
    int L;        // most tiles per workgroup
};

__device__ __forceinline__ PropTotals prop_totals(const int32_t *seq_lens, int B, int Hkv, int cap, int TT, long long P0,
                                                  int halve_long, int lane) {
    long long tiles = 0, nonempty = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int n = bb < B ? (clamp_len(seq_lens, bb, cap) + TT - 1) / TT : 0;
        tiles += wave_sum(n);
        nonempty += wave_sum(n > 0 ? 1 : 0);
    }
    const long long N = uniform64(tiles * Hkv), segs = uniform64(nonempty * Hkv);
    const long long P = shares_for(P0, N, segs, 0, halve_long);
    return PropTotals{N, N > 0 ? (int)((N + P - 1) / P) : 1};
}

// The piece of workgroup w: sequence b (< 0: none), kv head, split j of k, the
// sequence's (clamped) length.
struct PropPiece {
    int b, kvh, j, k, len;
};

__device__ __forceinline__ PropPiece prop_locate(const int32_t *seq_lens, int B, int Hkv, int cap, int TT, int L,
                                                 long long w, int lane) {
    PropPiece p{-1, 0, 0, 1, 0};
    long long run = 0;  // workgroups of the sequences before this chunk
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int ln = bb < B ? clamp_len(seq_lens, bb, cap) : 0;
        const int k = ((ln + TT - 1) / TT + L - 1) / L;  // 0 for an empty sequence
        const int cnt = k * Hkv;
        const int incl = wave_scan(cnt, lane);
        const unsigned long long hit = __ballot(bb < B && run + incl - cnt <= w && w < run + incl);
        if (p.b < 0 && hit != 0ull) {
            const int l = __builtin_ctzll(hit);
            p.b = c0 + l;
            p.k = __shfl(k, l, 64);
            p.len = __shfl(ln, l, 64);
            const long long r = w - (run + __shfl(incl - cnt, l, 64));
            p.kvh = (int)(r / p.k);
            p.j = (int)(r - (long long)p.kvh * p.k);
        }
        run += __shfl(incl, 63, 64);
    }
    p.b = __builtin_amdgcn_readfirstlane(p.b);
    p.kvh = __builtin_amdgcn_readfirstlane(p.kvh);
    p.j = __builtin_amdgcn_readfirstlane(p.j);
    p.k = __builtin_amdgcn_readfirstlane(p.k);
    p.len = __builtin_amdgcn_readfirstlane(p.len);
    return p;
}

// The first workgroup (slot) of sequence b's segments and its split count k.
__device__ __forceinline__ void prop_prefix(const int32_t *seq_lens, int B, int Hkv, int cap, int TT, int L, int b,
                                            int lane, long long &before, int &k_b) {
    long long pre = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int k = bb < B ? ((clamp_len(seq_lens, bb, cap) + TT - 1) / TT + L - 1) / L : 0;
        pre += wave_sum(bb < b ? k : 0);
    }
    before = uniform64(pre * Hkv);
    k_b = __builtin_amdgcn_readfirstlane(((clamp_len(seq_lens, b, cap) + TT - 1) / TT + L - 1) / L);
}

// Q of the R = M * G query rows of kv head kvh of sequence b (row r = i * G + g:
// query token i, head kvh * G + g), exact bf16, in the QK^T B operand layout.
// i = r / G by a multiply (qdiv = ceil(256 / G): exact for r, G <= 16); the
// row index fits 32 bits (B * M * Hq * D <= INT32_MAX, checked on the host).
// Columns r >= R load row R - 1 (no branch around the loads) and are zeroed.
template <int D, int KV>
__device__ __forceinline__ void load_q(const SplitArgs &a, int b, int kvh, int r, int grp,
                                       bf16x8_t (&qb)[Shape<D>::KB]) {
    const int rq = min(r, a.R - 1);
    const int qi = (rq * a.qdiv) >> 8;
    const int qg = rq - qi * a.G;
    const int qrow = ((b * a.M + qi) * a.Hq + kvh * a.G + qg) * D + kslot_lane<KV>(grp);
#pragma unroll
    for (int kb = 0; kb < Shape<D>::KB; ++kb) {
        u32x4_t x = *reinterpret_cast<const u32x4_t *>(a.q + qrow + kslot_block<KV>(kb));
        if (r >= a.R) x = u32x4_t{0u, 0u, 0u, 0u};
        qb[kb] = __builtin_bit_cast(bf16x8_t, x);
    }
}

// What a wave loads before its key range is known (see gqa_split_kernel).
template <int D, int NB, int KV>
struct Prefetch {
    Tile<D, NB, KV> tile;
    bf16x8_t qb[Shape<D>::KB];
};

// --------------------------------------------------------- one key range
//
// The workgroup's four waves process keys [t_begin, t_end) of segment
// (b, kvh), whose length is len: wave w takes tiles w, w+4, ..., each wave
// keeps its own (m, l, acc), and the waves are folded in ascending order
// through LDS into partial slot `slot` (or straight into `out` when direct).
// Must be called by all threads of the workgroup; ends with a barrier, after
// which LDS may be reused.  SPEC: Q and the wave's first tile are already in
// `pre`, the tile loaded against the cache capacity before the length was
// known (contiguous cache, single register tile only).  Paged: with have_pages,
// pages0 already holds the page ids of the wave's first 64 tiles (t_begin = 0).
template <int D, int NB, bool PAGED, int PV, bool DBUF, int CPOL, int KV, bool SPEC = false, int QKM = kQkMfma>
__device__ __forceinline__ void process_range(const SplitArgs &a, FoldLds<D, NB, QKM> &lds, int b, int kvh,
                                              int len, int t_begin, int t_end, size_t slot, bool direct,
                                              const Prefetch<D, NB, KV> *pre = nullptr, bool have_pages = false,
                                              int pages0 = 0) {
    static_assert(!SPEC || (!PAGED && !DBUF && PV == kPvBf16), "speculative first tile: default contiguous pipeline");
    using S = Shape<D>;
    constexpr int TT = 16 * NB;  // keys per wave tile
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int grp = lane >> 4;
    const int cap = PAGED ? a.max_pages * a.page_size : a.S_max;
    const int ntiles = t_end > t_begin ? (t_end - t_begin + TT - 1) / TT : 0;
    const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

    bf16x8_t qb[S::KB];
    if constexpr (SPEC) {
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) qb[kb] = pre->qb[kb];
    } else {
        load_q<D, KV>(a, b, kvh, r, grp, qb);
    }
    const unsigned *qtab = nullptr;
    float *xs = nullptr;
    if constexpr (QKM == kQkValu) {
        stage_q_valu<D>(qb, lds.qk.q[wave][0], r, grp);
        qtab = lds.qk.q[wave][0];
        xs = lds.qk.x[wave][0];
    }
    // Multi-query: query token i (row r = i * G + g) is position len - M + i
    // and sees keys < len - M + i + 1 (rows r >= R: any limit, never written).
    const int qi = (min(r, a.R - 1) * a.qdiv) >> 8;
    const int row_end = min(t_end, len - a.M + qi + 1);

    WaveState<D> st;
#pragma unroll
    for (int i = 0; i < S::NACC; ++i) st.acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;

    // Resources of the rows a tile reads.  Contiguous: the whole (b, kvh)
    // slab up to len.  Paged: the tile's page up to len (one table read).
    constexpr int EB = KV == kKvFp8 ? 1 : 2;  // bytes per cache element
    const size_t slab = (size_t)D * EB;       // bytes per row
    // Paged: lane i holds the page of this wave's tile (64*chunk + i), read
    // once per 64 tiles instead of one dependent scalar load per tile.
    int page_vec = 0;
    auto load_pages = [&](int chunk) {
        if constexpr (PAGED) {
            const int t0 = t_begin + (wave + kWaves * (64 * chunk + lane)) * TT;
            page_vec = 0;
            if (t0 < min(t_end, cap)) page_vec = a.page_table[(size_t)b * a.max_pages + t0 / a.page_size];
        }
    };
    if (have_pages) {
        page_vec = pages0;
    } else {
        load_pages(0);
    }
    auto issue = [&](Tile<D, NB, KV> &tile, int it, int parts) {
        const int t0 = t_begin + (wave + kWaves * it) * TT;
        if constexpr (PAGED) {
            if (it > 0 && (it & 63) == 0) load_pages(it >> 6);
            const int pidx = a.page_shift >= 0 ? t0 >> a.page_shift : t0 / a.page_size;
            const int row0 = t0 - pidx * a.page_size;
            const int page = min(max(__builtin_amdgcn_readlane(page_vec, it & 63), 0), a.num_pages - 1);
            const int rows = min(a.page_size, len - pidx * a.page_size);
            const size_t base = ((size_t)page * a.Hkv + kvh) * (size_t)a.page_size * slab;
            __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(a.k + base), (short)0, rows * D * EB, kRsrcWord3);
            __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(a.v + base), (short)0, rows * D * EB, kRsrcWord3);
            load_tile<D, NB, CPOL, KV>(tile, rk, rv, row0, r, grp, parts);
        } else {
            const size_t base = ((size_t)b * a.Hkv + kvh) * (size_t)a.S_max * slab;
            __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(a.k + base), (short)0, len * D * EB, kRsrcWord3);
            __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(a.v + base), (short)0, len * D * EB, kRsrcWord3);
            load_tile<D, NB, CPOL, KV>(tile, rk, rv, t0, r, grp, parts);
        }
    };
    auto tile_start = [&](int it) { return t_begin + (wave + kWaves * it) * TT; };

    unsigned short *stage = lds.stage(wave);
    if constexpr (DBUF) {
        // Two tile buffers: the next tile's loads are in flight during this tile's math.
        Tile<D, NB, KV> buf0, buf1;
        if (my_tiles > 0) issue(buf0, 0, kLoadK | kLoadV);
        for (int it = 0; it < my_tiles; it += 2) {
            if (it + 1 < my_tiles) issue(buf1, it + 1, kLoadK | kLoadV);
            compute_tile<D, NB, PV, KV>(buf0, qb, st, tile_start(it), row_end, r, grp, a.qk_scale_log2, stage);
            if (it + 1 < my_tiles) {
                if (it + 2 < my_tiles) issue(buf0, it + 2, kLoadK | kLoadV);
                compute_tile<D, NB, PV, KV>(buf1, qb, st, tile_start(it + 1), row_end, r, grp, a.qk_scale_log2, stage);
            }
        }
    } else {
        // One tile of registers, refilled as soon as each part is dead: the next
        // tile's K loads go out once QK^T has consumed K, its V loads once this
        // tile's V is in LDS, so they fly during the rest of the tile's math.
        // (Measured faster than two buffers or a ring of two tiles: the stream
        // is bandwidth-bound, and more loads in flight only add contention.)
        Tile<D, NB, KV> buf;
        if constexpr (SPEC) {
            buf = pre->tile;
        } else {
            if (my_tiles > 0) issue(buf, 0, kLoadV | kLoadK);
        }
        for (int it = 0; it < my_tiles; ++it) {
            const bool more = it + 1 < my_tiles;
            if constexpr (PV == kPvBf16) {
                f32x4_t sc[NB];
                if (it == 0) {
                    // The first tile's K arrives before its V (issued first):
                    // QK^T and the softmax run while V is still in flight.
                    qk_softmax<D, NB, KV, QKM>(buf, qb, st, tile_start(it), row_end, grp, a.qk_scale_log2, sc, qtab, xs, r, a.R);
                    if (more) issue(buf, it + 1, kLoadK);
                    if constexpr (SPEC) {
                        // rows past len were read from the capacity; K's are masked above
                        if (tile_start(it) + TT > len) zero_v_past(buf, tile_start(it), len, grp);
                    }
                    stage_v(buf, r, grp, stage);
                    if (more) issue(buf, it + 1, kLoadV);
                } else {
                    // Later tiles: stage V first, so that QK^T covers the LDS
                    // write latency before PV reads the staged V back.
                    stage_v(buf, r, grp, stage);
                    if (more) issue(buf, it + 1, kLoadV);
                    qk_softmax<D, NB, KV, QKM>(buf, qb, st, tile_start(it), row_end, grp, a.qk_scale_log2, sc, qtab, xs, r, a.R);
                    if (more) issue(buf, it + 1, kLoadK);
                }
                pv_tile<D, NB, PV, KV>(buf, sc, st, r, grp, stage);
            } else {
                compute_tile<D, NB, PV, KV>(buf, qb, st, tile_start(it), row_end, r, grp, a.qk_scale_log2, stage);
                if (more) issue(buf, it + 1, kLoadK | kLoadV);
            }
        }
    }

    // This wave's sum for head r: the four lanes r, r+16, r+32, r+48.
    const float lsum = sum_rows(st.l);

    // Publish the wave's state into its own region; rows r >= R are never read.
    if (r < a.R) {
        if (grp == 0) {
            lds.m[wave][r] = st.m;
            lds.l[wave][r] = lsum;
        }
        float *row = lds.acc(wave) + r * (D + 4);
        if constexpr (PV == kPvF32) {
#pragma unroll
            for (int c = 0; c < S::VC; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < S::DPL; e += 4) {
                        const f32x4_t x = {st.acc[c * S::DPL + e][i], st.acc[c * S::DPL + e + 1][i],
                                           st.acc[c * S::DPL + e + 2][i], st.acc[c * S::DPL + e + 3][i]};
                        *reinterpret_cast<f32x4_t *>(row + 16 * S::DPL * c + S::DPL * (4 * grp + i) + e) = x;
                    }
        } else {
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb)
                *reinterpret_cast<f32x4_t *>(row + 16 * nb + 4 * grp) = st.acc[nb];
        }
    }
    __syncthreads();

    // Fold the waves in ascending order: this range's partial (or the output).
    const int G = a.R;
    float *my_acc = a.part_acc + slot * G * D;
    float *my_ml = a.part_ml + slot * G * 2;
    for (int col = threadIdx.x; col < G * (D / 4); col += 64 * kWaves) {
        const int g = col / (D / 4);
        const int d = 4 * (col - g * (D / 4));
        // every LDS read of the column is issued before any is used
        float mw[kWaves], lw[kWaves];
        f32x4_t aw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = lds.m[w][g];
            lw[w] = lds.l[w][g];
            aw[w] = *reinterpret_cast<const f32x4_t *>(lds.acc(w) + g * (D + 4) + d);
        }
        float M = mw[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
        float L = 0.f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            // a wave without keys has m = -inf, l = 0 and a zero accumulator
            const float sw = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
            L += sw * lw[w];
            acc += sw * aw[w];
        }
        if constexpr (KV == kKvFp8) acc *= a.v_scale;  // the partials hold dequantised V sums
        if (direct) {
            const int i = g / a.G;  // row g = query token i, head kvh * G + (g - i * G)
            float *orow = a.out + (((size_t)b * a.M + i) * a.Hq + (size_t)kvh * a.G + (g - i * a.G)) * D;
            *reinterpret_cast<f32x4_t *>(orow + d) = L > 0.f ? acc / L : f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
            // Device-scope (write-through) stores: the combine kernel reads the
            // partials from other XCDs, and the kernel-end L2 writeback then has
            // nothing of them left to flush (measured faster hand-off).
            const __amdgpu_buffer_rsrc_t ra =
                __builtin_amdgcn_make_buffer_rsrc((void *)my_acc, (short)0, G * D * 4, kRsrcWord3);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc), ra, (g * D + d) * 4, 0, kDeviceScope);
            if (d == 0) {
                const __amdgpu_buffer_rsrc_t rm =
                    __builtin_amdgcn_make_buffer_rsrc((void *)my_ml, (short)0, G * 2 * 4, kRsrcWord3);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(M), __float_as_uint(L)}, rm, g * 8, 0,
                                                      kDeviceScope);
            }
        }
    }
    __syncthreads();
}

// --------------------------------------------------- one tile per wave
//
// A key range of at most four tiles (the short splits that fill the CUs for a
// single sequence): the four waves take one tile each and exchange, through
// LDS, first their score maxima, then their probabilities against the range's
// maximum (as bf16 hi + lo parts, each wave splitting only its own) and sums;
// each wave then computes PV over all four tiles for its own quarter of the
// head dims.  There is no fold of four accumulators afterwards: each wave
// writes its quarter of the range's partial (or of the output) straight from
// the MFMA registers.
//   m = max_w m_w,  P_w = 2^(S_w - m),  l = sum_w rowsum(P_w)  (ascending w),
//   acc[:, quarter] = sum_w P_w V_w[:, quarter]   (blocks of 16 keys in
//   ascending pairs, one 32-deep MFMA per pair and part).
// Tile loads as in process_range; `pf` holds Q and the tile when SPEC.
template <int D, int NB, bool PAGED, int CPOL, int KV, bool SPEC, int QKM = kQkMfma>
__device__ __forceinline__ void process_single(const SplitArgs &a, FoldLds<D, NB, QKM> &lds, int b, int kvh, int len,
                                               int t_begin, int t_end, size_t slot, bool direct,
                                               Prefetch<D, NB, KV> &pf) {
    constexpr int TT = 16 * NB;
    constexpr int NQ = D / 64;  // 16-dim blocks per quarter of the head dims
    constexpr int RS = kStageStride<D>;
    constexpr int EB = KV == kKvFp8 ? 1 : 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = lane & 15;
    const int grp = lane >> 4;
    const int t0 = t_begin + wave * TT;
    const bool has = t0 < t_end;  // this wave's tile holds keys of the range
    const int qi = (min(r, a.R - 1) * a.qdiv) >> 8;
    const int row_end = min(t_end, len - a.M + qi + 1);

    Tile<D, NB, KV> &tile = pf.tile;
    if constexpr (!SPEC) {
        load_q<D, KV>(a, b, kvh, r, grp, pf.qb);
        if (has) {
            if constexpr (PAGED) {
                const int pidx = t0 / a.page_size;
                const int page = min(max(a.page_table[(size_t)b * a.max_pages + pidx], 0), a.num_pages - 1);
                const int rows = min(a.page_size, len - pidx * a.page_size);
                const size_t base = ((size_t)page * a.Hkv + kvh) * (size_t)a.page_size * D * EB;
                const __amdgpu_buffer_rsrc_t rk =
                    __builtin_amdgcn_make_buffer_rsrc((void *)(a.k + base), (short)0, rows * D * EB, kRsrcWord3);
                const __amdgpu_buffer_rsrc_t rv =
                    __builtin_amdgcn_make_buffer_rsrc((void *)(a.v + base), (short)0, rows * D * EB, kRsrcWord3);
                load_tile<D, NB, CPOL, KV>(tile, rk, rv, t0 - pidx * a.page_size, r, grp, kLoadK | kLoadV);
            } else {
                const size_t base = ((size_t)b * a.Hkv + kvh) * (size_t)a.S_max * D * EB;
                const __amdgpu_buffer_rsrc_t rk =
                    __builtin_amdgcn_make_buffer_rsrc((void *)(a.k + base), (short)0, len * D * EB, kRsrcWord3);
                const __amdgpu_buffer_rsrc_t rv =
                    __builtin_amdgcn_make_buffer_rsrc((void *)(a.v + base), (short)0, len * D * EB, kRsrcWord3);
                load_tile<D, NB, CPOL, KV>(tile, rk, rv, t0, r, grp, kLoadK | kLoadV);
            }
        }
    }

    // This wave's scores (keys past the range or past a row's limit: -inf) and
    // their maximum per head row; the range's maximum is known after one exchange.
    f32x4_t sc[NB];
    float mx = -INFINITY;
    if constexpr (QKM == kQkValu) stage_q_valu<D>(pf.qb, lds.qk.q[wave][0], r, grp);
    if (has) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            f32x4_t c;
            if constexpr (QKM == kQkValu)
                c = qk_block<D, NB, KV, QKM>(tile, blk, pf.qb, lds.qk.q[wave][0], lds.qk.x[wave][0], r, grp, a.R);
            else
                c = qk_block<D, NB, KV, QKM>(tile, blk, pf.qb, nullptr, nullptr, r, grp, a.R);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = t0 + 16 * blk + 4 * grp + i;
                sc[blk][i] = tok < row_end ? c[i] * a.qk_scale_log2 : -INFINITY;
                mx = fmaxf(mx, sc[blk][i]);
            }
        }
        mx = max_rows(mx);
    } else {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) sc[blk] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    if (grp == 0) lds.m[wave][r] = mx;
    __syncthreads();

    // Probabilities against the range's maximum M (0 for a row with no key in
    // the range), published as bf16 hi + lo parts with this wave's sum; V staged.
    float M = lds.m[0][r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, lds.m[w][r]);
    const float m_ref = M == -INFINITY ? 0.f : M;
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        bf16x4_t hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[blk][i] - m_ref);
            psum += p;
            hi[i] = (__bf16)p;
            lo[i] = (__bf16)(p - (float)hi[i]);
        }
        const u32x2_t h = __builtin_bit_cast(u32x2_t, hi);
        const u32x2_t l = __builtin_bit_cast(u32x2_t, lo);
        lds.p[wave][blk][lane] = u32x4_t{h[0], h[1], l[0], l[1]};
    }
    const float lsum = sum_rows(psum);
    if (grp == 0) lds.l[wave][r] = lsum;
    unsigned short *stage = lds.stage(wave);
    if (has) {
        if (SPEC && t0 + TT > len) zero_v_past(tile, t0, len, grp);  // read against the capacity
    } else {
        zero_v_past(tile, t0, t0, grp);  // no keys: a zero V block meets zero probabilities
    }
    stage_v(tile, r, grp, stage);
    __syncthreads();

    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += lds.l[w][r];

    // PV over the range's 4 * NB blocks of 16 keys for this wave's quarter of
    // the dims, two blocks per 32-deep MFMA: contraction slots 8*grp .. + 3 hold
    // the first block's keys 4*grp .. + 3 and slots 8*grp + 4 .. + 7 the second
    // block's, in both operands (the lane's own probabilities and two
    // transposing reads), so no lane exchange is needed.  Every block takes part
    // (a tile without keys is all zeros), which lets all LDS reads go out at once.
    constexpr int NBLK = kWaves * NB;
    f32x4_t acc[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (a.R <= 8) {
        // At most 8 head rows: MFMA columns 8..15 carry the lo parts of rows
        // 0..7 (lane r >= 8 reads the lo half of lane r - 8's entry), so one
        // MFMA per pair takes both parts; each row's two column sums are added
        // once at the end (a row-of-16 rotation by 8).
        const int src = r < 8 ? lane : lane - 8;
        const int part = r < 8 ? 0 : 1;
#pragma unroll
        for (int e = 0; e < NBLK; e += 2) {
            u32x2_t pp[2];
            bf16x4_t av[2][NQ];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int w = (e + h) / NB;
                const int blk = (e + h) % NB;
                pp[h] = reinterpret_cast<const u32x2_t *>(&lds.p[w][blk][src])[part];
                const unsigned short *vsrc = lds.stage(w) + (16 * blk + 4 * grp + (r >> 2)) * RS + 4 * (r & 3);
#pragma unroll
                for (int j = 0; j < NQ; ++j)
                    av[h][j] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                                (lds_i16x4_t *)(vsrc + 16 * (wave * NQ + j))));
            }
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, u32x4_t{pp[0][0], pp[0][1], pp[1][0], pp[1][1]});
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const bf16x8_t v2 = __builtin_shufflevector(av[0][j], av[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, pb, acc[j], 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] += row_ror(acc[j][i], 8);
    } else {
#pragma unroll
        for (int e = 0; e < NBLK; e += 2) {
            u32x4_t pp[2];
            bf16x4_t av[2][NQ];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int w = (e + h) / NB;
                const int blk = (e + h) % NB;
                pp[h] = lds.p[w][blk][lane];
                const unsigned short *src = lds.stage(w) + (16 * blk + 4 * grp + (r >> 2)) * RS + 4 * (r & 3);
#pragma unroll
                for (int j = 0; j < NQ; ++j)
                    av[h][j] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                                (lds_i16x4_t *)(src + 16 * (wave * NQ + j))));
            }
            const bf16x8_t hi = __builtin_bit_cast(bf16x8_t, u32x4_t{pp[0][0], pp[0][1], pp[1][0], pp[1][1]});
            const bf16x8_t lo = __builtin_bit_cast(bf16x8_t, u32x4_t{pp[0][2], pp[0][3], pp[1][2], pp[1][3]});
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const bf16x8_t v2 = __builtin_shufflevector(av[0][j], av[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, hi, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, lo, acc[j], 0, 0, 0);
            }
        }
    }
    if constexpr (KV == kKvFp8) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) acc[j] *= a.v_scale;  // dequantised V sums
    }

    // Lane (r, grp) holds row r, dims 16*nb + 4*grp .. + 3 of each block nb.
    if (r < a.R) {
        const int G = a.R;
        if (direct) {
            const int i = r / a.G;  // row r = query token i, head kvh * G + (r - i * G)
            float *orow = a.out + (((size_t)b * a.M + i) * a.Hq + (size_t)kvh * a.G + (r - i * a.G)) * D;
#pragma unroll
            for (int j = 0; j < NQ; ++j)
                *reinterpret_cast<f32x4_t *>(orow + 16 * (wave * NQ + j) + 4 * grp) =
                    L > 0.f ? acc[j] / L : f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
            // device-scope stores, as in process_range
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.part_acc + slot * G * D), (short)0, G * D * 4, kRsrcWord3);
#pragma unroll
            for (int j = 0; j < NQ; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[j]), ra,
                                                       (r * D + 16 * (wave * NQ + j) + 4 * grp) * 4, 0, kDeviceScope);
            if (wave == 0 && grp == 0) {
                const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(a.part_ml + slot * G * 2), (short)0, G * 2 * 4, kRsrcWord3);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(M), __float_as_uint(L)}, rm, r * 8, 0,
                                                      kDeviceScope);
            }
        }
    }
}

// ------------------------------------------------------------ the fold
//
// The partials of one (sequence b, kv head) segment are folded with the
// log-sum-exp rescale (AstrAI csrc commit log, split-KV bullets; sparkinfer
// PR #877, section Mechanism), either by a combine kernel after the split
// kernel, or -- the in-kernel fold -- by the split workgroup that finishes a
// group of partials last, which it learns from an arrival ticket.

struct Fold {
    float m, l;
    f32x4_t o;
};

constexpr int kNarrowPieces = 16;  // partials loaded per round of a column fold

// One output column (4 dims of one row) over partials s = 0 .. n-1, where
// load(s) gives partial s's (m, l, 4 accumulator values), skipping the slots
// `skip(s)` names (a share that holds no tile writes nothing): rounds of
// kNarrowPieces partials in ascending order, each folded against the round's
// maximum.  The thread-per-column combine kernel and the in-kernel fold both
// call this, so the two give the same bits.
template <typename Load, typename Skip>
__device__ __forceinline__ Fold fold_column(int n, Load load, Skip skip) {
    float M = -INFINITY, L = 0.f;
    f32x4_t O = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += kNarrowPieces) {
        float mv[kNarrowPieces], lv[kNarrowPieces];
        f32x4_t av[kNarrowPieces];
        // Every load goes out before any is used (no branch around them):
        // slots past the last are read as the last one, and their values and
        // those of skipped slots are replaced by an empty partial.  The slot
        // flags are settled before the loads are issued: computed after them,
        // with a different segment per lane, the generated code (hipcc, ROCm
        // 7.2) flagged every slot after the first as skipped.
        bool used[kNarrowPieces];
#pragma unroll
        for (int u = 0; u < kNarrowPieces; ++u) used[u] = s0 + u < n && !skip(s0 + u);
        Fold x[kNarrowPieces];
#pragma unroll
        for (int u = 0; u < kNarrowPieces; ++u) x[u] = load(min(s0 + u, n - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kNarrowPieces; ++u) {
            mv[u] = used[u] ? x[u].m : -INFINITY;
            lv[u] = used[u] ? x[u].l : 0.f;
            av[u] = used[u] ? x[u].o : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        float mr = M;
#pragma unroll
        for (int u = 0; u < kNarrowPieces; ++u) mr = fmaxf(mr, mv[u]);
        if (mr != -INFINITY) {
            const float wr = __builtin_amdgcn_exp2f(M - mr);
            L *= wr;
            O *= wr;
#pragma unroll
            for (int u = 0; u < kNarrowPieces; ++u) {
                const float w = __builtin_amdgcn_exp2f(mv[u] - mr);
                L += w * lv[u];
                O += w * av[u];
            }
            M = mr;
        }
    }
    return Fold{M, L, O};
}

// Arrival counters of the in-kernel fold: the first kCounterBytes of the
// workspace, one 32-bit word per group of partials, zero between calls.
constexpr int kCounterBytes = 16384;
constexpr int kMaxCounters = kCounterBytes / 4;

// The ticket of a workgroup that has written its partial of a group of n:
// true for the last to arrive.  Every thread first waits until its own
// device-scope partial stores are complete, so when the last ticket is handed
// out every partial of the group is visible at device scope; the counter
// wraps back to zero on that last ticket (atomic increment modulo n), ready
// for the next call.  A vector (global) atomic; the result reaches the other
// threads through LDS.
__device__ __forceinline__ bool arrive_last(unsigned *ctr, int n, unsigned *lds_ticket) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
    __syncthreads();
    if (threadIdx.x == 0)
        *lds_ticket = __builtin_amdgcn_atomic_inc32(ctr, (unsigned)(n - 1), __ATOMIC_RELAXED, "agent");
    __syncthreads();
    const bool last = *lds_ticket == (unsigned)(n - 1);
    __syncthreads();  // the ticket word is free again
    return last;
}

// Nodes above the leaves of the fold tree over S partials with fan-in F
// (levels of ceil(n / F) nodes until one, the root, is left).
__host__ __device__ __forceinline__ int fold_tree_nodes(int S, int F) {
    int nodes = 0;
    for (int n = S; n > 1;) {
        n = (n + F - 1) / F;
        nodes += n;
    }
    return nodes;
}

// Even partition: slot s of a segment whose first piece is share w0 was
// written only if share w0 + s holds a tile (shares can be empty only when
// there are fewer positions than shares).
struct EmptyShareSkip {
    long long w0, N, P;
    bool maybe_empty;
    __device__ bool operator()(int s) const {
        return maybe_empty && share_begin(w0 + s, N, P) >= share_begin(w0 + s + 1, N, P);
    }
};

// In-kernel fold of one segment's partials (slots lo .. lo + n - 1, R rows
// each; with maybe_empty, slots of empty shares from w0 on are skipped as in
// EmptyShareSkip) by all threads of the workgroup: into the segment's output
// rows (final; row g = query token g / G, head kvh * G + g % G) or, as one
// more partial, into slot dst.  The partials were written by other
// workgroups of this launch: device-scope loads and stores.  Each split
// kernel calls it from one site (keeps the build small).
template <int D>
__device__ __forceinline__ void fold_segment(float *part_acc, float *part_ml, float *out, int R, int G, int M, int Hq,
                                          size_t lo, int n, long long w0, long long N, long long P, int maybe_empty,
                                          int b, int kvh, int final, size_t dst) {
    const EmptyShareSkip skip{w0, N, P, maybe_empty != 0};
    // Every column belongs to this segment: buffer resources on its first
    // slot (uniform), each lane's column as the offset.
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(part_ml + lo * R * 2), (short)0, n * R * 2 * 4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(part_acc + lo * R * D), (short)0, n * R * D * 4, kRsrcWord3);
    for (int col = threadIdx.x; col < R * (D / 4); col += 64 * kWaves) {
        const int g = col / (D / 4);
        const int d = 4 * (col - g * (D / 4));
        auto load = [&](int s) {
            const u32x2_t x = __builtin_bit_cast(
                u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, (s * R + g) * 8, 0, kDeviceScope));
            const f32x4_t v = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, ((s * R + g) * D + d) * 4, 0, kDeviceScope));
            return Fold{__uint_as_float(x[0]), __uint_as_float(x[1]), v};
        };
        const Fold f = fold_column(n, load, skip);
        if (final) {
            const int i = g / G;
            float *orow = out + (((size_t)b * M + i) * Hq + (size_t)kvh * G + (g - i * G)) * D;
            *reinterpret_cast<f32x4_t *>(orow + d) = f.l > 0.f ? f.o / f.l : f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(part_acc + dst * R * D), (short)0, R * D * 4, kRsrcWord3);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, f.o), ra, (g * D + d) * 4, 0,
                                                   kDeviceScope);
            if (d == 0) {
                const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(part_ml + dst * R * 2), (short)0, R * 2 * 4, kRsrcWord3);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(f.m), __float_as_uint(f.l)}, rm,
                                                      g * 8, 0, kDeviceScope);
            }
        }
    }
}

template <int D, int NB, bool PAGED, int PV, bool DBUF, int PART, int CPOL, int KV, int QKM = kQkMfma>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kMinWavesPerEu<D, NB, DBUF>)))
void gqa_split_kernel(const int32_t *seq_lens, const unsigned char *k, const unsigned char *v, const uint16_t *q,
                      int num_splits, int Hkv, int B, int cap, int split_tokens, int qpack, const SplitArgs args) {
    constexpr int TT = 16 * NB;
    __shared__ FoldLds<D, NB, QKM> lds;
    // The leading scalar arguments arrive preloaded in SGPRs, so the length,
    // Q and first-tile loads below issue without waiting for the kernel-argument
    // fetch.  qpack = G | M << 5 | R << 10 | qdiv << 15.
    SplitArgs a = args;
    a.seq_lens = seq_lens;
    a.k = k;
    a.v = v;
    a.q = q;
    a.num_splits = num_splits;
    a.Hkv = Hkv;
    a.B = B;
    a.split_tokens = split_tokens;
    a.G = qpack & 31;
    a.M = (qpack >> 5) & 31;
    a.R = (qpack >> 10) & 31;
    a.qdiv = qpack >> 15;
    a.Hq = Hkv * a.G;

    if constexpr (PART == kPartitionEven) {
        const int lane = threadIdx.x & 63;
        if (args.prop) {
            // Proportional splits: this workgroup's one piece (the partial goes
            // to slot blockIdx.x; the combine kernel folds each segment's k).
            const long long P0 = (long long)gridDim.x - (long long)a.B * a.Hkv;
            const PropTotals tot = prop_totals(a.seq_lens, a.B, a.Hkv, cap, TT, P0, a.halve_long, lane);
            const PropPiece pc = prop_locate(a.seq_lens, a.B, a.Hkv, cap, TT, tot.L, blockIdx.x, lane);
            if (pc.b < 0) return;
            const int n = (pc.len + TT - 1) / TT;
            const int tb = (int)((long long)pc.j * n / pc.k);
            const int te = (int)((long long)(pc.j + 1) * n / pc.k);
            process_range<D, NB, PAGED, PV, DBUF, CPOL, KV, false, QKM>(a, lds, pc.b, pc.kvh, pc.len, tb * TT,
                                                                        min(pc.len, te * TT), (size_t)blockIdx.x, false);
            return;
        }
        // This workgroup's equal share of the tile axis (each segment's tiles
        // plus K positions for its start and fold), walked piece by piece.
        const int K = a.piece_cost;
        // In-kernel fold: no piece covers a sequence of length 0, so the
        // workgroups zero its output rows (sequences blockIdx.x, + grid, ...).
        auto zero_empty = [&]() {
            if (!args.fused) return;
            for (int bb = blockIdx.x; bb < a.B; bb += gridDim.x) {
                if (__builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens, bb, cap)) != 0) continue;
                f32x4_t *o = reinterpret_cast<f32x4_t *>(a.out + (size_t)bb * a.M * a.Hq * D);
                for (int i = threadIdx.x; i < a.M * a.Hq * (D / 4); i += 64 * kWaves) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        };
        SegmentLocation loc;
        long long cur, end, P;
        if (a.B <= 64) {
            // one load of the lengths: the total, then this share's start
            const int ln = lane < a.B ? clamp_len(a.seq_lens, lane, cap) : 0;
            const int n = seg_span((ln + TT - 1) / TT, K);
            const int incl = wave_scan(n, lane);
            const long long N = uniform64((long long)__shfl(incl, 63, 64) * a.Hkv);
            const long long segs = uniform64((long long)wave_sum(ln > 0 ? 1 : 0) * a.Hkv);
            P = shares_for(gridDim.x, N, segs, K, a.halve_long);
            if ((long long)blockIdx.x >= P) return zero_empty();
            cur = share_begin(blockIdx.x, N, P);
            end = share_begin(blockIdx.x + 1, N, P);
            if (cur >= end) return zero_empty();
            const unsigned long long hit =
                __ballot(lane < a.B && (long long)(incl - n) * a.Hkv <= cur && cur < (long long)incl * a.Hkv);
            const int l = __builtin_ctzll(hit);
            loc.total = N;
            loc.b = __builtin_amdgcn_readfirstlane(l);
            loc.len = __builtin_amdgcn_readfirstlane(__shfl(ln, l, 64));
            loc.before = uniform64((long long)__shfl(incl - n, l, 64) * a.Hkv);
        } else {
            loc = locate_tile(a.seq_lens, a.B, a.Hkv, cap, TT, K, -1, lane);  // the total only
            const long long segs = a.halve_long ? nonempty_segments(a.seq_lens, a.B, a.Hkv, cap, lane) : 0;
            P = shares_for(gridDim.x, loc.total, segs, K, a.halve_long);
            if ((long long)blockIdx.x >= P) return zero_empty();
            cur = share_begin(blockIdx.x, loc.total, P);
            end = share_begin(blockIdx.x + 1, loc.total, P);
            if (cur >= end) return zero_empty();
            loc = locate_tile(a.seq_lens, a.B, a.Hkv, cap, TT, K, cur, lane);
        }
        int b = loc.b;
        int len = loc.len;
        int nb_tiles = (len + TT - 1) / TT;  // tiles of the segment; it spans nb_tiles + K positions
        const int rel = (int)(cur - loc.before);  // < Hkv * (nb_tiles + K)
        int kvh = __builtin_amdgcn_readfirstlane(rel / (nb_tiles + K));
        int off = __builtin_amdgcn_readfirstlane(rel - kvh * (nb_tiles + K));
        // Paged: a share that runs on into the next segment (tile 0 of
        // (b, kvh + 1) or (b + 1, 0)) loads that segment's length and the page
        // ids of its first tiles when the current piece starts, so that the
        // next piece's first loads do not wait for them (measured: 3% faster on
        // batches of short paged sequences; no gain, and a loss, contiguous).
        bool have_pages = false;
        int pages = 0;
        // In-kernel fold: a segment this share covers whole is written to
        // `out` directly; the (at most two) segments it shares with other
        // workgroups take their arrival tickets once the share is done, so the
        // stream never stalls on them, and the last piece to arrive folds.
        const long long N = loc.total;
        struct Pending {
            int b, kvh, n, arrivals;
            long long w0;
        };
        Pending pend0{}, pend1{};
        int npend = 0;
        // Only the segments holding the share's first and last positions can
        // extend beyond it (a segment inside the share is held by it alone),
        // so a share has at most two such pieces pending.
        auto settle = [&]() {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are done
            __syncthreads();
            if (threadIdx.x == 0) {
                lds.ticket[0] = __builtin_amdgcn_atomic_inc32(args.counters + (size_t)pend0.b * a.Hkv + pend0.kvh,
                                                              (unsigned)(pend0.arrivals - 1), __ATOMIC_RELAXED, "agent");
                if (npend > 1)
                    lds.ticket[1] = __builtin_amdgcn_atomic_inc32(args.counters + (size_t)pend1.b * a.Hkv + pend1.kvh,
                                                                  (unsigned)(pend1.arrivals - 1), __ATOMIC_RELAXED,
                                                                  "agent");
            }
            __syncthreads();
            const unsigned t0 = lds.ticket[0], t1 = lds.ticket[1];
            __syncthreads();  // the ticket words are free again
#pragma unroll 1
            for (int i = 0; i < npend; ++i) {  // one call site of the fold
                const Pending p = i == 0 ? pend0 : pend1;
                if ((i == 0 ? t0 : t1) != (unsigned)(p.arrivals - 1)) continue;
                fold_segment<D>(a.part_acc, a.part_ml, a.out, a.R, a.G, a.M, a.Hq,
                                (size_t)p.w0 + (size_t)p.b * a.Hkv + p.kvh, p.n, p.w0, N, P, N < P, p.b, p.kvh, 1, 0);
            }
        };
        while (cur < end) {
            // off < nb_tiles + K here
            const bool same_b = kvh + 1 < a.Hkv;
            const int nb = same_b ? b : b + 1;
            int next_len = 0;
            int next_pages = 0;
            bool fetched = false;  // next_len / next_pages were loaded for segment (nb, ...)
            if (off < nb_tiles) {
                const int take = (int)min((long long)(nb_tiles - off), end - cur);
                const size_t slot = (size_t)blockIdx.x + (size_t)b * a.Hkv + kvh;
                bool whole = false;  // in-kernel fold: this piece is the whole segment
                if (args.fused) {
                    // the segment's tiles are axis positions [z, z + nb_tiles), held by shares w0 .. w1
                    const long long z = cur - off;
                    const long long w0 = share_of(z, N, P);
                    const int npieces = (int)(share_of(z + nb_tiles - 1, N, P) - w0 + 1);
                    if (npieces == 1) {
                        whole = true;
                    } else {
                        int arrivals = npieces;  // shares holding a tile (only those write a piece)
                        if (N < P)
                            for (int i = 0; i < npieces; ++i)
                                arrivals -= share_begin(w0 + i, N, P) >= share_begin(w0 + i + 1, N, P) ? 1 : 0;
                        const Pending pe{b, kvh, npieces, arrivals, w0};
                        if (npend == 0) pend0 = pe;
                        else pend1 = pe;
                        ++npend;
                    }
                }
                const bool has_next = off + take == nb_tiles && cur + take + K < end;
                if (PAGED && has_next) {
                    next_len = same_b ? len : load_len_or_zero(a.seq_lens, nb, a.B);
                    next_pages = load_page_or_zero(a.page_table, nb,
                                                   ((int)(threadIdx.x >> 6) + kWaves * lane) * TT / a.page_size, a.B,
                                                   a.max_pages);
                    fetched = true;
                }
                process_range<D, NB, PAGED, PV, DBUF, CPOL, KV, false, QKM>(a, lds, b, kvh, len, off * TT,
                                                                min(len, (off + take) * TT), slot, whole, nullptr,
                                                                have_pages, pages);
                cur += take;
                off += take;
            }
            have_pages = false;
            if (off >= nb_tiles) {  // the segment's tiles are done: step over its K positions
                cur += nb_tiles + K - off;
                off = nb_tiles + K;
            }
            if (cur < end) {
                off = 0;
                const int nlen = fetched ? min(max(__builtin_amdgcn_readfirstlane(next_len), 0), cap) : 0;
                if (nlen > 0) {  // the segment loaded ahead
                    b = nb;
                    kvh = same_b ? kvh + 1 : 0;
                    len = nlen;
                    pages = next_pages;
                    have_pages = true;
                } else if (++kvh == a.Hkv) {
                    kvh = 0;
                    do {  // sequences of length 0 hold no tiles
                        ++b;
                        len = b < a.B ? __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens, b, cap)) : 1;
                    } while (len == 0);
                }
                nb_tiles = (len + TT - 1) / TT;
            }
        }
        if (npend > 0) settle();
        return zero_empty();
    } else {
        const int b = blockIdx.x / (num_splits * Hkv);  // one division before the length load
        const int len_v = load_len_vmem(seq_lens, b);
        __builtin_amdgcn_sched_barrier(0);  // the length load goes out first
        const int bk = blockIdx.x / num_splits;
        const int split = blockIdx.x - bk * num_splits;
        const int kvh = bk - b * Hkv;
        const int t_begin = split * a.split_tokens;
        const int nsplit = a.num_splits;
        const bool direct = nsplit == 1;
        // Contiguous cache: the wave's first tile does not wait for the length.
        // It is loaded against the capacity (rows below S_max are the caller's
        // memory) while the length is in flight; rows past the length are
        // masked (K) and zeroed (V) once it is known.
        constexpr bool kSpec = !PAGED && !DBUF && PV == kPvBf16;
        Prefetch<D, NB, KV> pre;
        if constexpr (kSpec) {
            // No branch around the loads (so the wait for the length does not
            // wait for them too): a tile at or past the capacity reads zeros
            // through the buffer bounds, and its offsets stay below
            // (S_max + 64) * D * bytes, which fits 32 bits.
            constexpr int EB = KV == kKvFp8 ? 1 : 2;
            const int t0 = t_begin + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * TT;
            const int lane = threadIdx.x & 63;
            load_q<D, KV>(a, b, kvh, lane & 15, lane >> 4, pre.qb);
            const size_t base = ((size_t)b * a.Hkv + kvh) * (size_t)cap * D * EB;
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void *)(a.k + base), (short)0, cap * D * EB, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void *)(a.v + base), (short)0, cap * D * EB, kRsrcWord3);
            load_tile<D, NB, CPOL, KV>(pre.tile, rk, rv, t0, lane & 15, lane >> 4, kLoadK | kLoadV);
            __builtin_amdgcn_sched_barrier(0);  // ... and goes out before the wait for the length
        }
        // Out-of-range lengths / page ids are clamped so that no access can leave
        // the caller's buffers (the results for such inputs are unspecified).
        const int len = min(max(__builtin_amdgcn_readfirstlane(len_v), 0), cap);
        const int t_end = min(len, t_begin + a.split_tokens);
        const size_t slot = (size_t)bk * nsplit + split;
        // (the one-tile path splits the head dims in quarters of 16-dim blocks: D >= 64)
        if (D >= 64 && !DBUF && PV == kPvBf16 && a.split_tokens <= kWaves * TT) {
            if constexpr (D >= 64)
                process_single<D, NB, PAGED, CPOL, KV, kSpec, QKM>(a, lds, b, kvh, len, t_begin, t_end, slot, direct,
                                                                   pre);
        } else {
            process_range<D, NB, PAGED, PV, DBUF, CPOL, KV, kSpec, QKM>(a, lds, b, kvh, len, t_begin, t_end, slot,
                                                                        direct, &pre);
        }
        if (args.fused && !direct) {
            // In-kernel fold: a tree over the segment's splits, fan-in F.  The
            // last of a node's children to arrive folds them (in ascending
            // order) into the node's partial, then arrives at the parent; the
            // root's folder writes the output.  Node j of a level has the
            // children F*j .. F*j + F - 1 of the level below; level slots and
            // counters follow the splits' partials, level after level.
            const int F = args.fanin;
            const int nodes = fold_tree_nodes(nsplit, F);
            unsigned *ctr = args.counters + bk * nodes;
            const size_t tree = (size_t)a.B * a.Hkv * nsplit + bk * (size_t)(nodes - 1);
            size_t child0 = bk * (size_t)nsplit;  // slot of node 0 of the current level
            int level_n = nsplit, j = split, off = 0;
            while (true) {
                const int parent = j / F;
                const int first = parent * F;
                const int cnt = min(F, level_n - first);
                const int next_n = (level_n + F - 1) / F;
                if (!arrive_last(ctr + off + parent, cnt, &lds.ticket[0])) break;
                const bool root = next_n == 1;
                fold_segment<D>(a.part_acc, a.part_ml, a.out, a.R, a.G, a.M, a.Hq, child0 + first, cnt, 0, 0, 1, 0, b,
                                kvh, root, tree + off + parent);
                if (root) break;
                child0 = tree + off;
                off += next_n;
                level_n = next_n;
                j = parent;
            }
        }
    }
}

// Combine: one workgroup of 256 threads per (b, h, chunk of 4*NCOL dims).
// Thread (sg, c), c = tid % NCOL, owns dims 4c .. 4c+3 of the chunk and the
// pieces s with s % NSG == sg (NSG = 256 / NCOL).  It loads U of its pieces
// at a time and folds each round into its running (m, l, o) against the
// round's maximum (independent exponentials, not a chain of merges).  The
// NSG folds of a column are then combined max first inside each wave: the
// wave's maximum for the column (a max tree over the lanes that share c: row
// rotations, then the row-pair and half-wave swaps), each fold rescaled once to
// it, and the rescaled (l, o) summed by the same tree; the four waves' results
// then meet in LDS (one barrier) and the column's thread merges them in wave
// order against their common maximum.  Every step has a fixed order, so the
// result is bit-reproducible.
constexpr int kCombineThreads = 256;

template <int NCOL, int PART>
__global__ __launch_bounds__(kCombineThreads) void gqa_combine_kernel(const float *part_acc, const float *part_ml,
                                                                        int num_splits, int G_arg, int Hq, int D_arg,
                                                                        const CombineArgs args) {
    // leading scalar arguments: preloaded in SGPRs (the partial loads wait on nothing else)
    CombineArgs a = args;
    a.part_acc = part_acc;
    a.part_ml = part_ml;
    a.num_splits = num_splits;
    a.G = G_arg;
    a.Hq = Hq;
    a.D = D_arg;
    static_assert(NCOL == 2 || NCOL == 4 || NCOL == 8 || NCOL == 16, "lanes of one column must share rows of 16");
    constexpr int NSG = kCombineThreads / NCOL;
    constexpr int U = 4;  // pieces per thread per round of loads
    const int D = a.D;
    const int chunks = D / (4 * NCOL);
    const size_t bh = blockIdx.x / chunks;
    const int d0 = (blockIdx.x % chunks) * 4 * NCOL;
    const int c = threadIdx.x % NCOL;
    const int sg = threadIdx.x / NCOL;
    const int G = a.G;
    const size_t b = bh / a.Hq;
    const int h = (int)(bh % a.Hq);
    const size_t bk = b * (a.Hq / G) + h / G;   // segment b * Hkv + kvh
    const int g = h % G;
    // The segment's partials are the consecutive slots [lo, lo + S); slot k of
    // head g: acc at (k*G + g)*D, ml at (k*G + g)*2.
    size_t lo;
    int S;
    long long N = 0, P = 1, w0 = 0;  // even partition: slot lo + s belongs to share w0 + s
    bool maybe_empty = false;         // shares can be empty only when there are fewer tiles than shares
    if constexpr (PART == kPartitionFixed) {
        S = a.num_splits;
        lo = bk * S;
    } else {
        long long before, total;
        const int lane = threadIdx.x & 63;
        long long segs;
        prefix_tiles(a.seq_lens, a.B, a.Hkv, a.cap, a.tile, a.piece_cost, (int)b, lane, before, total, segs);
        const int n = (clamp_len(a.seq_lens, (int)b, a.cap) + a.tile - 1) / a.tile;
        N = total;
        P = shares_for(a.shares, N, segs, a.piece_cost, a.halve_long);
        maybe_empty = N < P;
        if (n == 0) {
            S = 0;
            lo = 0;
        } else {
            // the segment's tiles are axis positions [z, z + n) (its K extra ones follow)
            const long long z = before + (long long)(h / G) * seg_span(n, a.piece_cost);
            w0 = share_of(z, N, P);
            S = (int)(share_of(z + n - 1, N, P) - w0 + 1);
            lo = (size_t)(w0 + (long long)bk);
        }
    }
    const float *ml = a.part_ml + (lo * G + g) * 2;
    const float *acc = a.part_acc + (lo * G + g) * D + d0 + 4 * c;
    const size_t ml_stride = (size_t)G * 2, acc_stride = (size_t)G * D;

    Fold run{-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
    for (int s0 = sg; s0 < S; s0 += U * NSG) {
        float mv[U], lv[U];
        f32x4_t av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * NSG;
            mv[u] = -INFINITY;
            lv[u] = 0.f;
            av[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // even partition: a share that holds no tile wrote nothing
            const bool used = !maybe_empty || share_begin(w0 + s, N, P) < share_begin(w0 + s + 1, N, P);
            if (s < S && used) {
                mv[u] = ml[s * ml_stride];
                lv[u] = ml[s * ml_stride + 1];
                av[u] = *reinterpret_cast<const f32x4_t *>(acc + s * acc_stride);
            }
        }
        float mr = run.m;
#pragma unroll
        for (int u = 0; u < U; ++u) mr = fmaxf(mr, mv[u]);
        if (mr != -INFINITY) {
            const float wr = __builtin_amdgcn_exp2f(run.m - mr);
            run.l *= wr;
            run.o *= wr;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float w = __builtin_amdgcn_exp2f(mv[u] - mr);
                run.l += w * lv[u];
                run.o += w * av[u];
            }
            run.m = mr;
        }
    }

    // The wave's maximum for column c: lanes of one column inside a wave are c,
    // c + NCOL, ... (64 / NCOL of them).
    __shared__ float wm[kWaves][NCOL], wl[kWaves][NCOL];
    __shared__ f32x4_t wo[kWaves][NCOL];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float mx = run.m;
    if constexpr (NCOL <= 2) mx = fmaxf(mx, row_ror(mx, 2));
    if constexpr (NCOL <= 4) mx = fmaxf(mx, row_ror(mx, 4));
    if constexpr (NCOL <= 8) mx = fmaxf(mx, row_ror(mx, 8));
    {
        LanePair q = rows16(mx);
        q = halves32(fmaxf(q.lo, q.hi));
        mx = fmaxf(q.lo, q.hi);
    }

    // Each fold rescaled to the wave's maximum once (an empty fold, m = -inf,
    // weighs 0), then the sums by the same tree; the four waves' (max, sums)
    // meet in LDS and are merged in wave order by the column's thread.
    const float wt = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(run.m - mx);
    float sl = run.l * wt;
    f32x4_t so = run.o * wt;
    auto add_ror = [&](int n) {
        sl += row_ror(sl, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) so[i] += row_ror(so[i], n);
    };
    if constexpr (NCOL <= 2) add_ror(2);
    if constexpr (NCOL <= 4) add_ror(4);
    if constexpr (NCOL <= 8) add_ror(8);
    auto add_swap = [&](auto pair) {
        LanePair q = pair(sl);
        sl = q.lo + q.hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q = pair(so[i]);
            so[i] = q.lo + q.hi;
        }
    };
    add_swap([](float v) { return rows16(v); });
    add_swap([](float v) { return halves32(v); });
    if (lane < NCOL) {
        wm[wave][lane] = mx;
        wl[wave][lane] = sl;
        wo[wave][lane] = so;
    }
    __syncthreads();
    if (threadIdx.x < NCOL) {
        float M = wm[0][c];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w][c]);
        float L = 0.f;
        f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float ww = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm[w][c] - M);
            L += ww * wl[w][c];
            O += ww * wo[w][c];
        }
        // row h = kvh * G + i * Gh + gh of sequence b is out[b][i][kvh * Gh + gh]
        size_t orow = bh;
        if (a.M > 1) {
            const int rho = h % G, i = rho / a.Gh;
            orow = ((size_t)b * a.M + i) * (size_t)(a.Hq / a.M) + (size_t)(h / G) * a.Gh + (rho - i * a.Gh);
        }
        *reinterpret_cast<f32x4_t *>(a.out + orow * D + d0 + 4 * c) =
            L > 0.f ? O / L : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
}

// Combine for plans whose segments have few pieces (even shares of a batch,
// a few fixed splits): one thread per (output row, 4 dims).  Each wave takes
// 64 consecutive columns of one sequence; a thread loads the pieces of its
// column kNarrowPieces at a time (one round when the segment has no more) and
// folds each round in ascending order against the round's maximum.  No tree,
// no LDS, no barrier.
constexpr int kNarrowThreads = 64;  // one wave per workgroup: the waves spread over every CU

template <int PART>
__global__ __launch_bounds__(kNarrowThreads) void gqa_combine_narrow_kernel(const float *part_acc,
                                                                               const float *part_ml, int num_splits,
                                                                               int G_arg, int Hq, int D_arg,
                                                                               const CombineArgs args) {
    CombineArgs a = args;
    a.part_acc = part_acc;
    a.part_ml = part_ml;
    a.num_splits = num_splits;
    a.G = G_arg;
    a.Hq = Hq;
    a.D = D_arg;
    const int D = a.D;
    const int cols = a.Hq * (D / 4);  // columns of one sequence
    const int waves_per_b = (cols + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x;
    const int b = __builtin_amdgcn_readfirstlane(wave / waves_per_b);
    if (b >= a.B) return;  // the whole wave
    const int col = (wave - b * waves_per_b) * 64 + lane;
    const bool active = col < cols;
    const int h = active ? col / (D / 4) : 0;
    const int d = 4 * (col - h * (D / 4));
    const int G = a.G;
    const size_t bk = (size_t)b * (a.Hq / G) + h / G;  // segment b * Hkv + kvh
    const int g = h % G;
    size_t lo;
    int S;
    long long N = 0, P = 1, w0 = 0;
    bool maybe_empty = false;
    if constexpr (PART == kPartitionFixed) {
        S = a.num_splits;
        lo = bk * S;
    } else if (a.prop) {
        // proportional splits: sequence b's segments hold k consecutive slots each
        const PropTotals tot = prop_totals(a.seq_lens, a.B, a.Hkv, a.cap, a.tile, a.shares, a.halve_long, lane);
        long long before;
        int k;
        prop_prefix(a.seq_lens, a.B, a.Hkv, a.cap, a.tile, tot.L, b, lane, before, k);
        S = k;
        lo = (size_t)(before + (long long)(h / G) * k);
    } else {
        long long before, total;
        long long segs;
        prefix_tiles(a.seq_lens, a.B, a.Hkv, a.cap, a.tile, a.piece_cost, b, lane, before, total, segs);
        const int n = (clamp_len(a.seq_lens, b, a.cap) + a.tile - 1) / a.tile;
        N = total;
        P = shares_for(a.shares, N, segs, a.piece_cost, a.halve_long);
        maybe_empty = N < P;
        if (n == 0) {
            S = 0;
            lo = 0;
        } else {
            // the segment's tiles are axis positions [z, z + n) (its K extra ones follow)
            const long long z = before + (long long)(h / G) * seg_span(n, a.piece_cost);
            w0 = share_of(z, N, P);
            S = (int)(share_of(z + n - 1, N, P) - w0 + 1);
            lo = (size_t)(w0 + (long long)bk);
        }
    }
    if (!active) S = 0;
    const float *ml = a.part_ml + (lo * G + g) * 2;
    const float *acc = a.part_acc + (lo * G + g) * D + d;
    const size_t ml_stride = (size_t)G * 2, acc_stride = (size_t)G * D;
    auto load = [&](int s) {
        const u32x2_t x = *reinterpret_cast<const u32x2_t *>(ml + s * ml_stride);
        return Fold{__uint_as_float(x[0]), __uint_as_float(x[1]), *reinterpret_cast<const f32x4_t *>(acc + s * acc_stride)};
    };
    const Fold f = fold_column(S, load, EmptyShareSkip{w0, N, P, maybe_empty});
    const float L = f.l;
    const f32x4_t O = f.o;
    if (!active) return;
    // row h = kvh * G + i * Gh + gh of sequence b is out[b][i][kvh * Gh + gh]
    size_t orow = (size_t)b * a.Hq + h;
    if (a.M > 1) {
        const int rho = h % G, i = rho / a.Gh;
        orow = ((size_t)b * a.M + i) * (size_t)(a.Hq / a.M) + (size_t)(h / G) * a.Gh + (rho - i * a.Gh);
    }
    *reinterpret_cast<f32x4_t *>(a.out + orow * D + d) = L > 0.f ? O / L : f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ host side

constexpr int kMaxDevices = 64;
constexpr int kDefaultPieceCost = 4;
constexpr int kDefaultSplitKeys = 2048;
std::atomic<int> g_cu_count[kMaxDevices];

// ------------------------------------------------------------------ launches
//
// Kernels are launched through the module API with their function handles
// looked up once per (kernel, device): hipLaunchKernelGGL resolves the handle
// on every launch, which costs about half a microsecond of host time per
// launch (measured on MI355X), and a call's host time bounds callers that do
// not replay graphs.
std::mutex g_func_mu;
std::unordered_map<uint64_t, hipFunction_t> g_funcs;  // key: kernel address * kMaxDevices + device

hipError_t function_of(const void *kernel, hipFunction_t *f) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    const uint64_t key = (uint64_t)(uintptr_t)kernel * kMaxDevices + (uint64_t)dev;
    std::lock_guard<std::mutex> lock(g_func_mu);
    const auto it = g_funcs.find(key);
    if (it != g_funcs.end()) {
        *f = it->second;
        return hipSuccess;
    }
    e = hipGetFuncBySymbol(f, kernel);
    if (e == hipSuccess) {
        try {
            g_funcs.emplace(key, *f);
        } catch (...) {  // nothing throws across the C ABI; the handle is still valid
        }
    }
    return e;
}

template <typename... P, typename... A, size_t... I>
hipError_t launch_indexed(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, std::index_sequence<I...>,
                          A &&...args) {
    // each argument converted to its parameter's exact type, then passed by address
    std::tuple<std::decay_t<P>...> values(std::forward<A>(args)...);
    void *params[] = {static_cast<void *>(&std::get<I>(values))...};
    hipFunction_t f = nullptr;
    const hipError_t e = function_of(reinterpret_cast<const void *>(kernel), &f);
    if (e != hipSuccess) return e;
    return hipModuleLaunchKernel(f, grid.x, grid.y, grid.z, block.x, block.y, block.z, 0, stream, params, nullptr);
}

template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "one value per kernel parameter");
    return launch_indexed(kernel, grid, block, stream, std::index_sequence_for<P...>{}, std::forward<A>(args)...);
}

// ------------------------------------------------------------------ tuning
//
// The plan and kernel-variant choices every call makes, process-wide.  The
// defaults are the measured best on MI355X; GQA_DECODE_* environment variables
// override them for same-binary A/B runs, read once when the library is
// loaded; gqa_decode_set_tuning replaces the whole set at run time.  Every
// call copies the tuning once at entry, so the kernels of one call, and the
// plan they derive, always agree.
gqa_tuning_t default_tuning() {
    gqa_tuning_t t{};
    t.pv_mode = 1;  // kPvBf16
    t.streaming = 1;
    t.piece_cost = kDefaultPieceCost;
    t.halve_long = 1;
    return t;
}

bool tuning_valid(const gqa_tuning_t &t) {
    auto in = [](int v, int lo, int hi) { return v >= lo && v <= hi; };
    return (t.tile_tokens == 0 || t.tile_tokens == 16 || t.tile_tokens == 32 || t.tile_tokens == 64) &&
           in(t.double_buffer, 0, 1) && in(t.pv_mode, 0, 1) && in(t.streaming, 0, 1) && in(t.partition, 0, 3) &&
           in(t.shares, 0, INT32_MAX / 2) && in(t.split_keys, 0, INT32_MAX) && in(t.piece_cost, 0, 1024) &&
           in(t.halve_long, 0, 1) && in(t.combine, 0, 1) &&
           (t.combine_cols == 0 || t.combine_cols == 2 || t.combine_cols == 4 || t.combine_cols == 8 ||
            t.combine_cols == 16) &&
           in(t.num_splits, 0, INT32_MAX) && in(t.fold, 0, 2) && in(t.qk_mode, 0, 1);
}

// Each variable that is set to a valid value replaces its field; anything
// else leaves the default.
gqa_tuning_t tuning_from_env() {
    gqa_tuning_t t = default_tuning();
    auto num = [](const char *name, int &field, int lo, int hi) {
        const char *s = getenv(name);
        if (s == nullptr || *s == '\0') return;
        char *end = nullptr;
        const long v = strtol(s, &end, 10);
        if (*end == '\0' && v >= lo && v <= hi) field = (int)v;
    };
    auto is = [](const char *name, const char *value) {
        const char *s = getenv(name);
        return s != nullptr && strcmp(s, value) == 0;
    };
    int tile = 0, cols = 0;
    num("GQA_DECODE_TILE", tile, 16, 64);
    if (tile == 16 || tile == 32 || tile == 64) t.tile_tokens = tile;
    if (is("GQA_DECODE_DBUF", "1")) t.double_buffer = 1;
    if (is("GQA_DECODE_PV", "f32")) t.pv_mode = 0;
    if (is("GQA_DECODE_NT", "0")) t.streaming = 0;
    if (is("GQA_DECODE_PARTITION", "fixed")) t.partition = 1;
    if (is("GQA_DECODE_PARTITION", "even")) t.partition = 2;
    if (is("GQA_DECODE_PARTITION", "prop")) t.partition = 3;
    num("GQA_DECODE_SHARES", t.shares, 1, INT32_MAX / 2);
    num("GQA_DECODE_SPLIT_KEYS", t.split_keys, 1, INT32_MAX);
    num("GQA_DECODE_PIECE_COST", t.piece_cost, 0, 1024);
    if (is("GQA_DECODE_HALVE_LONG", "0")) t.halve_long = 0;
    if (is("GQA_DECODE_COMBINE", "tree")) t.combine = 1;
    num("GQA_DECODE_COMBINE_COLS", cols, 2, 16);
    if (cols == 2 || cols == 4 || cols == 8 || cols == 16) t.combine_cols = cols;
    num("GQA_DECODE_SPLITS", t.num_splits, 1, INT32_MAX);
    if (is("GQA_DECODE_FOLD", "kernel")) t.fold = 1;
    if (is("GQA_DECODE_FOLD", "fused")) t.fold = 2;
    if (is("GQA_DECODE_QK", "valu")) t.qk_mode = 1;
    return t;
}

std::mutex g_tuning_mu;
gqa_tuning_t g_tuning = tuning_from_env();  // dynamic initialisation: once, at load

gqa_tuning_t current_tuning() {
    std::lock_guard<std::mutex> lock(g_tuning_mu);
    return g_tuning;
}

// Keys per wave tile: 16 KB of K+V per wave (64 keys at D=64, 32 at D=128,
// 16 at D=256).  A tuned tile (16, 32 or 64) replaces it when the result
// stays within 16 KB.
int tile_tokens_for(int D, bool double_buffer, bool paged, int elem_bytes, int tuned) {
    int dflt = double_buffer ? (D <= 64 ? 64 : (D == 128 ? 32 : 16)) : (D == 32 ? 64 : (D == 64 ? 32 : 16));
    // A paged E4M3 cache at head_dim 128: 32 keys, so that a wave still reads
    // 4 KB of K (and of V) in one piece of a page, as a bf16 tile of 16 does
    // (measured: the ragged 8k paged workload 80.2 -> 62.4 us per call).
    if (!double_buffer && paged && elem_bytes == 1 && D == 128) dflt = 32;
    if (tuned != 0 && tuned * D <= 4096) return tuned;
    return dflt;
}

bool supported_dim(int D) { return D == 32 || D == 64 || D == 128 || D == 256; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

gqa_status_t device_cu_count(int *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return GQA_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
        return GQA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
    *out = c;
    return GQA_OK;
}

struct WorkspaceLayout {
    size_t counters, part_acc, part_ml, total;
};

// The arrival counters of the in-kernel fold first (kCounterBytes, in every
// plan's workspace, so that calls of any shape can share one workspace without
// a partial ever landing on a counter), then `slots` partial blocks of G
// heads: B*Hkv*S (+ the fold tree's nodes) for fixed splits, P + B*Hkv for P
// even shares.
WorkspaceLayout workspace_layout(int Hq, int Hkv, int D, int64_t slots) {
    WorkspaceLayout w{};
    const size_t G = (size_t)(Hq / Hkv);
    size_t off = 0;
    w.counters = off;
    off += kCounterBytes;
    w.part_acc = off;
    off += align_up((size_t)slots * G * D * sizeof(float), 256);
    w.part_ml = off;
    off += align_up((size_t)slots * G * 2 * sizeof(float), 256);
    w.total = off;
    return w;
}

// Which plans fold in the split kernel by default (tuning fold = 0).  On
// MI355X a level of the in-kernel fold costs more than the second launch it
// saves unless the fold is small: the device-scope store acknowledgement and
// the ticket take ~1.3 us, and one workgroup folding a group is held to a
// single CU's memory pipe, where the combine kernel spreads the same reads
// over the whole device.  Measured, us per call (two launches vs one): GQA-6
// hd256 4k 8.6 vs 15.1, 128k keys on one kv head 16.2 vs 20.4, ragged paged 8k
// 107.6 vs 111.3, uniform 16k batch 83.0 vs 82.6 -- but 512 keys on two kv
// heads in 4 splits 6.18 vs 5.61 (2, 4 and 8 splits all favour one launch).
// So fixed splits fold in the kernel when the whole fold is one small node
// (at most kNarrowPieces partials, kSmallFoldBytes in all, per segment),
// and everything else folds in a combine kernel.
constexpr bool kFuseEvenByDefault = false;
constexpr int64_t kSmallFoldBytes = 16 << 10;

// Fan-in of the fold tree over S fixed splits: one node for up to
// kNarrowPieces splits, else the smallest power of two F with F * F >= S
// (at most kNarrowPieces): two levels up to 256 splits.
int fold_fanin(int S) {
    if (S <= kNarrowPieces) return S;
    int F = 2;
    while (F * F < S && F < kNarrowPieces) F *= 2;
    return F;
}

// Even shares over a contiguous bf16 cache: whether the kernels may take one
// share per CU when the segments are long (decided on the device from
// seq_lens, the same way in the split and combine kernels).  Off for paged
// caches, for E4M3 caches (half the bytes per tile for the same math: their
// second workgroup per CU hides it; measured 50.2 -> 62.0 us per call at the
// batched E4M3 workload with one per CU), and when the tuning fixes the share
// count or turns the rule off.
int halve_long_shares(const gqa_tuning_t &t, bool paged, int kv) {
    return (!paged && kv == kKvBf16 && t.shares == 0 && t.halve_long) ? 1 : 0;
}

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

hipError_t launch_combine(const gqa_plan_t &plan, const gqa_tuning_t &t, const float *part_acc,
                          const float *part_ml, float *out, const int32_t *seq_lens, int B, int M, int Hq, int Hkv,
                          int D, int cap, int halve_long, hipStream_t stream) {
    // rows: M query tokens x Hq heads per sequence, M * G per (sequence, kv head)
    const int rows = M * Hq;
    const bool prop = plan.partition == kPartitionProp;
    // the split kernel's share count: the launched grid, less one workgroup per segment for proportional splits
    const int shares = prop ? plan.grid - B * Hkv : plan.grid;
    CombineArgs ca{part_acc, part_ml, out, seq_lens, D, rows / Hkv, rows, plan.num_splits,
                   B, Hkv, cap, plan.tile_tokens, shares, M, Hq / Hkv, t.piece_cost, halve_long, prop ? 1 : 0};
    // The widest dim chunk (NCOL = 16, 8, 4 or 2 columns of 4 dims) that
    // still gives at least 128 workgroups: narrower chunks put more threads on
    // the pieces of a column (measured best for few heads with many pieces).
    // The tuning's combine_cols (2, 4, 8 or 16) overrides it.
    const int64_t heads = (int64_t)B * rows;
    const bool even = plan.partition == kPartitionEven || prop;
    // Few pieces per segment (at full length): one thread per column folds
    // them (no tree).  The tuning's combine = 1 keeps the tree for A/B runs.
    // Proportional splits always take the thread-per-column combine.
    if ((t.combine == 0 && plan.max_pieces <= kNarrowPieces) || prop) {
        const int64_t waves = (int64_t)B * ((rows * (D / 4) + 63) / 64);
        auto go = [&](auto kernel) {
            return launch(kernel, dim3((unsigned)waves), dim3(kNarrowThreads), stream, ca.part_acc, ca.part_ml,
                          ca.num_splits, ca.G, ca.Hq, ca.D, ca);
        };
        return even ? go(gqa_combine_narrow_kernel<kPartitionEven>) : go(gqa_combine_narrow_kernel<kPartitionFixed>);
    }
    int ncol = t.combine_cols;
    if (ncol != 2 && ncol != 4 && ncol != 8 && ncol != 16) {
        ncol = 16;
        while (ncol > 2 && heads * (D / (4 * ncol)) < 128) ncol /= 2;
    }
    while (4 * ncol > D) ncol /= 2;  // a chunk never exceeds the head (head_dim 32: 8 columns)
    const unsigned grid = (unsigned)(heads * (D / (4 * ncol)));
    auto go = [&](auto kernel) {
        return launch(kernel, dim3(grid), dim3(kCombineThreads), stream, ca.part_acc, ca.part_ml, ca.num_splits, ca.G,
                      ca.Hq, ca.D, ca);
    };
    if (ncol == 16) return even ? go(gqa_combine_kernel<16, kPartitionEven>) : go(gqa_combine_kernel<16, kPartitionFixed>);
    if (ncol == 8) return even ? go(gqa_combine_kernel<8, kPartitionEven>) : go(gqa_combine_kernel<8, kPartitionFixed>);
    if (ncol == 4) return even ? go(gqa_combine_kernel<4, kPartitionEven>) : go(gqa_combine_kernel<4, kPartitionFixed>);
    return even ? go(gqa_combine_kernel<2, kPartitionEven>) : go(gqa_combine_kernel<2, kPartitionFixed>);
}

template <int D, int NB, bool PAGED>
hipError_t launch_split_nb(const gqa_plan_t &plan, const SplitArgs &a, int kv, hipStream_t stream) {
    if constexpr (NB * D > 256) {  // at most 16 KB of K+V (64 * NB * D bytes) per wave tile
        return hipErrorInvalidValue;
    } else {
        const dim3 grid((unsigned)plan.grid), block(64 * kWaves);
        const int cap = PAGED ? a.max_pages * a.page_size : a.S_max;
        const bool even = plan.partition == kPartitionEven || plan.partition == kPartitionProp;
        const bool nt = plan.streaming != 0;
        const int qpack = a.G | a.M << 5 | a.R << 10 | a.qdiv << 15;  // each field <= 16, qdiv <= 256
        hipError_t err = hipErrorInvalidValue;  // stays so if no branch below launches
        auto go = [&](auto kernel) {
            err = launch(kernel, grid, block, stream, a.seq_lens, a.k, a.v, a.q, a.num_splits, a.Hkv, a.B, cap,
                         a.split_tokens, qpack, a);
        };
        if (kv == kKvFp8) {
            // The E4M3 cache always runs the default pipeline (bf16 PV, one register tile);
            // its 16-byte K loads feed two 32-dim k-blocks, so it needs D >= 64.
            if constexpr (D < 64) {
                return hipErrorInvalidValue;
            } else {
                if (nt) even ? go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionEven, kNonTemporal, kKvFp8>)
                             : go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionFixed, kNonTemporal, kKvFp8>);
                else even ? go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionEven, 0, kKvFp8>)
                          : go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionFixed, 0, kKvFp8>);
            }
        } else if (D >= 64 && plan.pv_mode == kPvF32) {  // (its fold reads 4 dims per lane: D >= 64)
            if constexpr (D >= 64) {
                even ? go(gqa_split_kernel<D, NB, PAGED, kPvF32, true, kPartitionEven, 0, kKvBf16>)
                     : go(gqa_split_kernel<D, NB, PAGED, kPvF32, true, kPartitionFixed, 0, kKvBf16>);
            }
        } else if (plan.double_buffer) {
            even ? go(gqa_split_kernel<D, NB, PAGED, kPvBf16, true, kPartitionEven, 0, kKvBf16>)
                 : go(gqa_split_kernel<D, NB, PAGED, kPvBf16, true, kPartitionFixed, 0, kKvBf16>);
        } else if (nt && plan.qk_mode == kQkValu) {
            if constexpr (D >= 128 && NB == 1) {
                even ? go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionEven, kNonTemporal, kKvBf16, kQkValu>)
                     : go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionFixed, kNonTemporal, kKvBf16, kQkValu>);
            } else {
                return hipErrorInvalidValue;  // the plan never selects it here
            }
        } else if (nt) {
            even ? go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionEven, kNonTemporal, kKvBf16>)
                 : go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionFixed, kNonTemporal, kKvBf16>);
        } else {
            even ? go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionEven, 0, kKvBf16>)
                 : go(gqa_split_kernel<D, NB, PAGED, kPvBf16, false, kPartitionFixed, 0, kKvBf16>);
        }
        return err;
    }
}

template <int D, bool PAGED>
hipError_t launch_split(const gqa_plan_t &plan, const SplitArgs &a, int kv, hipStream_t stream) {
    switch (plan.tile_tokens) {
        case 16: return launch_split_nb<D, 1, PAGED>(plan, a, kv, stream);
        case 32: return launch_split_nb<D, 2, PAGED>(plan, a, kv, stream);
        case 64: return launch_split_nb<D, 4, PAGED>(plan, a, kv, stream);
        default: return hipErrorInvalidValue;
    }
}

constexpr int kPhaseSplit = 1;
constexpr int kPhaseCombine = 2;

// Element type and per-tensor scales of the cache of one call.
struct KvSpec {
    int type;       // kKvBf16 or kKvFp8
    float k_scale;  // E4M3 only
    float v_scale;
};
constexpr KvSpec kBf16Cache{kKvBf16, 1.f, 1.f};

gqa_status_t run(const gqa_plan_t &plan, const gqa_tuning_t &t, SplitArgs &a, int D, bool paged, int kv,
                 void *workspace, hipStream_t stream, int phases) {
    a.piece_cost = t.piece_cost;
    a.halve_long = halve_long_shares(t, paged, kv);
    if (!plan.direct) {
        WorkspaceLayout w = workspace_layout(a.M * a.Hq, a.Hkv, D, plan.slots);
        char *base = static_cast<char *>(workspace);
        a.counters = reinterpret_cast<unsigned *>(base + w.counters);
        a.part_acc = reinterpret_cast<float *>(base + w.part_acc);
        a.part_ml = reinterpret_cast<float *>(base + w.part_ml);
    }
    // Only a whole call folds in the split kernel: a *_partials call leaves
    // every partial for gqa_decode_combine.
    a.fused = plan.fused && phases == (kPhaseSplit | kPhaseCombine) ? 1 : 0;
    a.fanin = plan.fold_fanin;
    a.prop = plan.partition == kPartitionProp ? 1 : 0;
    hipError_t e = hipSuccess;
    if (phases & kPhaseSplit) {
        switch (D) {
            case 32: e = paged ? launch_split<32, true>(plan, a, kv, stream) : launch_split<32, false>(plan, a, kv, stream); break;
            case 64: e = paged ? launch_split<64, true>(plan, a, kv, stream) : launch_split<64, false>(plan, a, kv, stream); break;
            case 128: e = paged ? launch_split<128, true>(plan, a, kv, stream) : launch_split<128, false>(plan, a, kv, stream); break;
            case 256: e = paged ? launch_split<256, true>(plan, a, kv, stream) : launch_split<256, false>(plan, a, kv, stream); break;
            default: return GQA_ERR_UNSUPPORTED;
        }
        if (e != hipSuccess) return GQA_ERR_HIP;
    }
    if (plan.direct || !(phases & kPhaseCombine) || a.fused) return GQA_OK;
    const int cap = paged ? a.max_pages * a.page_size : a.S_max;
    e = launch_combine(plan, t, a.part_acc, a.part_ml, a.out, a.seq_lens, a.B, a.M, a.Hq, a.Hkv, D, cap,
                       a.halve_long, stream);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status_t check_common(const void *q, const void *k, const void *v, const int32_t *seq_lens,
                          const float *out, int B, int Hq, int Hkv, int D, float scale) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !isfinite(scale)) return GQA_ERR_SHAPE;
    if (!supported_dim(D) || Hq / Hkv > kMaxHeadsPerKv) return GQA_ERR_UNSUPPORTED;
    if (B == 0) return GQA_OK;  // nothing is read or written
    if (!q || !k || !v || !seq_lens || !out) return GQA_ERR_NULL;
    if ((int64_t)B * Hq * D > INT32_MAX) return GQA_ERR_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(seq_lens, 4))
        return GQA_ERR_ALIGN;
    return GQA_OK;
}

gqa_status_t plan_impl(int B, int Hq, int Hkv, int D, int max_seq_len, int page_size, int num_splits,
                       int cu_count, int elem_bytes, const gqa_tuning_t &t, gqa_plan_t *plan);

// elem_bytes: 2 for a bf16 cache, 1 for E4M3.
gqa_status_t plan_for_call(int B, int Hq, int Hkv, int D, int cap, int page_size, int num_splits,
                           const gqa_tuning_t &t, gqa_plan_t *plan, int elem_bytes = 2) {
    if (num_splits == 0) num_splits = t.num_splits;
    int cu = 256;
    if (num_splits == 0) {
        gqa_status_t s = device_cu_count(&cu);
        if (s != GQA_OK) return s;
    }
    return plan_impl(B, Hq, Hkv, D, cap, page_size, num_splits, cu, elem_bytes, t, plan);
}

}  // namespace

extern "C" {

// The plan a call with these arguments makes (the tuning's num_splits applies
// when num_splits is 0, as in a call).
gqa_status_t gqa_decode_plan(int B, int Hq, int Hkv, int D, int max_seq_len, int page_size,
                             int num_splits, int cu_count, gqa_plan_t *plan) {
    const gqa_tuning_t t = current_tuning();
    return plan_impl(B, Hq, Hkv, D, max_seq_len, page_size, num_splits == 0 ? t.num_splits : num_splits, cu_count,
                     2, t, plan);
}

gqa_status_t gqa_decode_plan_fp8(int B, int Hq, int Hkv, int D, int max_seq_len, int page_size,
                                 int num_splits, int cu_count, gqa_plan_t *plan) {
    const gqa_tuning_t t = current_tuning();
    return plan_impl(B, Hq, Hkv, D, max_seq_len, page_size, num_splits == 0 ? t.num_splits : num_splits, cu_count,
                     1, t, plan);
}

void gqa_decode_get_tuning(gqa_tuning_t *tuning) {
    if (tuning != nullptr) *tuning = current_tuning();
}

gqa_status_t gqa_decode_set_tuning(const gqa_tuning_t *tuning) {
    if (tuning == nullptr) return GQA_ERR_NULL;
    if (!tuning_valid(*tuning)) return GQA_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_tuning_mu);
    g_tuning = *tuning;
    return GQA_OK;
}

}  // extern "C"

namespace {

gqa_status_t plan_impl(int B, int Hq, int Hkv, int D, int max_seq_len, int page_size, int num_splits,
                       int cu_count, int elem_bytes, const gqa_tuning_t &t, gqa_plan_t *plan) {
    if (plan == nullptr) return GQA_ERR_NULL;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_seq_len < 0 || page_size < 0 ||
        num_splits < 0 || cu_count <= 0)
        return GQA_ERR_SHAPE;
    if (!supported_dim(D) || Hq / Hkv > kMaxHeadsPerKv) return GQA_ERR_UNSUPPORTED;
    if (page_size > 0 && page_size % 16 != 0) return GQA_ERR_UNSUPPORTED;

    *plan = gqa_plan_t{};
    const int dbuf = t.double_buffer;
    int tt = tile_tokens_for(D, dbuf != 0, page_size > 0, elem_bytes, t.tile_tokens);
    if (page_size > 0) {
        while (page_size % tt != 0) tt /= 2;  // a tile never straddles a page (tt >= 16)
    }
    int tiles_total = max_seq_len > 0 ? (max_seq_len + tt - 1) / tt : 1;
    const int base = B > 0 ? B * Hkv : 1;
    const bool want_fixed = t.partition == 1;
    const bool want_even = t.partition == 2;
    const bool want_prop = t.partition == 3;

    // Small jobs: one 16-key tile per wave in fixed splits.  `most16` is the
    // split count that gives every wave one 16-key tile at full length.
    //  - A batch whose splits so cut take at most four workgroups per CU runs
    //    them instead of even shares: the share walk needs the lengths before
    //    its first tile load (a dependent round trip) and runs the multi-tile
    //    loop, which a small job cannot amortise (us per call, fixed vs even:
    //    2 x 4 kv heads x 1024 keys 6.96 vs 10.32; 8 x 1 x 512 7.31 vs 11.46;
    //    4 x 8 x 1024 8.91 vs 12.55; ragged 8 x 8 x 1..1024 12.96 vs 13.54;
    //    past four per CU the even shares win on ragged batches: 16 x 8 x
    //    1..1024 18.72 vs 15.92).
    //  - Where the default tile is longer (head_dim 32 and 64), a fixed plan
    //    within half the device takes 16-key tiles, twice the workgroups
    //    (512 keys on two kv heads at head_dim 64: 5.29 vs 5.74; 4096 keys at
    //    head_dim 32: 5.39 vs 5.95).
    const bool auto_tile = t.tile_tokens == 0 && !dbuf;
    const int64_t most16 = max_seq_len > 0 ? ((int64_t)(max_seq_len + 15) / 16 + kWaves - 1) / kWaves : 0;
    bool small_fixed = false;
    if (auto_tile && num_splits == 0 && t.partition == 0 && B > 1 && tiles_total > 4 * kWaves && most16 >= 2 &&
        (int64_t)base * most16 <= 4 * (int64_t)cu_count) {
        small_fixed = true;
    }
    const bool fixed_by_shape = !(tiles_total > 4 * kWaves && (B > 1 || want_even || want_prop));
    if (auto_tile && num_splits == 0 && tt > 16 && most16 >= 2 &&
        (small_fixed || (fixed_by_shape && (int64_t)base * most16 <= cu_count / 2))) {
        tt = 16;
        tiles_total = (max_seq_len + tt - 1) / tt;
        small_fixed = true;  // one tile per wave (the doubled tile count must not turn a batch to shares)
    }
    plan->tile_tokens = tt;
    plan->waves = kWaves;
    plan->pv_mode = t.pv_mode;
    plan->double_buffer = dbuf;
    // Non-temporal K/V loads: every KV byte is read once per call, and in a
    // decode step the caches of all layers together far exceed the 256 MB
    // Infinity Cache, so they stream from HBM (measured faster at every
    // workload size when the inputs are not cache-resident).
    plan->streaming = t.streaming;
    // QK^T on the vector ALU (A/B variant): the default pipeline only, head_dim
    // 128 or 256 with 16-key tiles, bf16 cache.
    plan->qk_mode = (t.qk_mode == kQkValu && elem_bytes == 2 && D >= 128 && tt == 16 && !dbuf && t.pv_mode == kPvBf16 &&
                     t.streaming) ? kQkValu : kQkMfma;

    // Even shares (the default for batches): about two workgroups per CU, each at least
    // one tile per wave at full length; a segment short enough for one
    // workgroup (<= 4 tiles per wave) is written directly instead.
    // A single sequence cannot be ragged: fixed splits give it the same work
    // split without the device-side length scan.
    if (num_splits == 0 && !want_fixed && !small_fixed && tiles_total > 4 * kWaves &&
        (B > 1 || want_even || want_prop)) {
        const int64_t tiles_max = (int64_t)base * tiles_total;
        int64_t P = t.shares > 0 ? t.shares : (B > 1 ? 2 * cu_count : cu_count);
        if (P > (tiles_max + kWaves - 1) / kWaves) P = (tiles_max + kWaves - 1) / kWaves;
        if (P < 1) P = 1;
        if (P > INT32_MAX / 2) return GQA_ERR_SHAPE;
        if (want_prop) {
            // Proportional splits: P workgroups' worth of at most L tiles each
            // (decided on the device from seq_lens), plus up to one more per
            // segment for the rounding of each segment's split count.
            const int64_t L = (tiles_max + P - 1) / P;  // at full length, P not halved
            if (P + base > INT32_MAX / 2) return GQA_ERR_SHAPE;
            plan->partition = kPartitionProp;
            plan->num_splits = 0;
            plan->split_tokens = (int)std::min<int64_t>(L * tt, INT32_MAX);
            plan->grid = B > 0 ? (int)(P + base) : 0;
            plan->direct = 0;
            plan->slots = P + base;
            plan->max_pieces = (int)std::min<int64_t>(P, (tiles_total + L - 1) / L);
            plan->workspace_bytes = workspace_layout(Hq, Hkv, D, plan->slots).total;
            return GQA_OK;
        }
        plan->partition = kPartitionEven;
        plan->num_splits = 0;
        plan->split_tokens = (int)((tiles_max + P - 1) / P) * tt;  // keys per share at full length
        plan->grid = B > 0 ? (int)P : 0;
        plan->direct = 0;
        plan->slots = (int64_t)P + base;
        // Pieces of one segment with every sequence at full length: its tiles
        // span positions of shares of about N / P positions (N = the segments'
        // tiles plus K each), so at most floor((tiles - 1) * P / N) + 2 shares.
        // Shorter sequences elsewhere make shares shorter and can give a
        // segment more pieces; the combine walks them all either way.
        const int64_t N_full = (int64_t)base * (tiles_total + (t.piece_cost >= 0 ? t.piece_cost : 0));
        plan->max_pieces =
            (int)std::min<int64_t>(std::min<int64_t>(P, tiles_total), ((int64_t)(tiles_total - 1) * P) / N_full + 2);
        // In-kernel fold: one counter per (sequence, kv head); every segment's
        // few pieces are folded by the share that finishes last among them.
        // Not for segments of many pieces (one workgroup would read them all).
        const bool fuse = t.fold == 2 || (t.fold == 0 && kFuseEvenByDefault && plan->max_pieces <= kNarrowPieces);
        if (fuse && base <= kMaxCounters) {
            plan->fused = 1;
            plan->counters = base;
        }
        plan->workspace_bytes = workspace_layout(Hq, Hkv, D, plan->slots).total;
        return GQA_OK;
    }

    // Fixed splits: enough workgroups to give every CU one of them (measured
    // best for one long sequence: fewer partials to fold, no loss in the
    // stream), and no split longer than the tuning's split_keys (2048 keys),
    // but at least one tile per wave; a short segment (<= 4 tiles per wave)
    // gets a single split.
    const int kMaxSplitTokens = t.split_keys > 0 ? t.split_keys : kDefaultSplitKeys;
    int S = num_splits;
    if (S == 0 && small_fixed) {
        S = (int)most16;  // one tile per wave
    } else if (S == 0) {
        const int fill = (cu_count + base - 1) / base;
        const int len_cap = (max_seq_len + kMaxSplitTokens - 1) / kMaxSplitTokens;
        S = fill > len_cap ? fill : len_cap;
        const int most = (tiles_total + kWaves - 1) / kWaves;
        if (S > most) S = most;
        if (tiles_total <= 4 * kWaves) {
            // A short segment fits one workgroup (a direct write), but while
            // the splits take at most half the device, one tile per wave over
            // several workgroups and a small fold finish sooner (cold caches,
            // us per call, direct vs split: 512 keys on two kv heads 7.00 vs
            // 5.63; 256 keys on 8 kv heads 6.73 vs 6.27; GQA-6 hd256 with 256
            // keys 10.85 vs 7.64; with the splits filling every CU, 64 kv
            // heads of 256 keys: 7.02 vs 7.59).
            S = (most >= 2 && (int64_t)base * most <= cu_count / 2) ? most : 1;
        }
    }
    if (S > tiles_total) S = tiles_total;
    if (S < 1) S = 1;
    int split_tiles = (tiles_total + S - 1) / S;
    S = (tiles_total + split_tiles - 1) / split_tiles;  // drop splits that would be empty

    plan->partition = kPartitionFixed;
    plan->num_splits = S;
    plan->split_tokens = split_tiles * tt;
    const int64_t grid = (int64_t)(B > 0 ? B : 0) * Hkv * S;
    if (grid > INT32_MAX) return GQA_ERR_SHAPE;
    plan->grid = (int)grid;
    plan->direct = S == 1 ? 1 : 0;
    plan->slots = (int64_t)base * S;
    plan->max_pieces = S;
    plan->workspace_bytes = 0;
    if (!plan->direct) {
        // In-kernel fold: a tree over each segment's splits (fan-in F), one
        // counter per node; the inner nodes' partials follow the splits'.
        const bool small = S <= kNarrowPieces && (int64_t)S * (Hq / Hkv) * D * 4 <= kSmallFoldBytes;
        const bool fuse = t.fold == 2 || (t.fold == 0 && small);
        const int F = fold_fanin(S);
        const int64_t nodes = fold_tree_nodes(S, F);
        if (fuse && (int64_t)base * nodes <= kMaxCounters) {
            plan->fused = 1;
            plan->fold_fanin = F;
            plan->counters = (int64_t)base * nodes;
            plan->slots += (int64_t)base * (nodes - 1);
        }
        plan->workspace_bytes = workspace_layout(Hq, Hkv, D, plan->slots).total;
    }
    return GQA_OK;
}

}  // namespace

extern "C" {

// The bf16 plan: an upper bound for an E4M3 cache too (its longer paged tiles
// give no more shares or splits).
size_t gqa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_seq_len, int page_size,
                                  int num_splits) {
    gqa_plan_t plan;
    if (plan_for_call(B, Hq, Hkv, D, max_seq_len, page_size, num_splits, current_tuning(), &plan) != GQA_OK)
        return SIZE_MAX;
    return plan.workspace_bytes;
}

}  // extern "C"

namespace {

// Checks of the query-token count M (1 for single-token decode): M * G query
// rows per kv head must fit the 16 MFMA columns.
gqa_status_t check_queries(int B, int M, int Hq, int Hkv, int D) {
    if (M < 1) return GQA_ERR_SHAPE;
    if (Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && (int64_t)M * (Hq / Hkv) > kMaxHeadsPerKv)
        return GQA_ERR_UNSUPPORTED;
    if ((int64_t)B * M * Hq * D > INT32_MAX) return GQA_ERR_SHAPE;
    return GQA_OK;
}

gqa_status_t decode_contig(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, int B, int M, int Hq, int Hkv, int D, int S_max,
                           float scale, const KvSpec &kv, float *out, void *workspace,
                           size_t workspace_bytes, int num_splits, hipStream_t stream, int phases) {
    gqa_status_t s = check_common(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, scale);
    if (s != GQA_OK) return s;
    if (kv.type == kKvFp8 && D < 64) return GQA_ERR_UNSUPPORTED;  // E4M3: head_dim 64, 128 or 256
    if ((s = check_queries(B, M, Hq, Hkv, D)) != GQA_OK) return s;
    if (S_max < 0 || num_splits < 0 || !isfinite(kv.k_scale) || !isfinite(kv.v_scale)) return GQA_ERR_SHAPE;
    if (B == 0) return GQA_OK;
    const int eb = kv.type == kKvFp8 ? 1 : 2;
    if (((int64_t)S_max + 64) * D * eb > INT32_MAX) return GQA_ERR_SHAPE;  // 32-bit buffer offsets
    if (workspace != nullptr && misaligned(workspace, 16)) return GQA_ERR_ALIGN;
    const gqa_tuning_t t = current_tuning();
    gqa_plan_t plan;
    s = plan_for_call(B, M * Hq, Hkv, D, S_max, 0, num_splits, t, &plan, kv.type == kKvFp8 ? 1 : 2);
    if (s != GQA_OK) return s;
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return workspace == nullptr ? GQA_ERR_NULL : GQA_ERR_WORKSPACE;
    if (B == 0) return GQA_OK;
    SplitArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const unsigned char *>(k_cache);
    a.v = static_cast<const unsigned char *>(v_cache);
    a.seq_lens = seq_lens;
    a.out = out;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.M = M; a.R = M * (Hq / Hkv); a.qdiv = (256 + a.G - 1) / a.G;
    a.S_max = S_max;
    a.num_splits = plan.num_splits;
    a.split_tokens = plan.split_tokens;
    a.qk_scale_log2 = scale * kv.k_scale * 1.4426950408889634f;
    a.v_scale = kv.v_scale;
    return run(plan, t, a, D, false, kv.type, workspace, stream, phases);
}

gqa_status_t decode_paged(const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *seq_lens, const int32_t *page_table, int B, int M, int Hq,
                          int Hkv, int D, int page_size, int num_pages, int max_pages,
                          float scale, const KvSpec &kv, float *out, void *workspace,
                          size_t workspace_bytes, int num_splits, hipStream_t stream, int phases) {
    gqa_status_t s = check_common(q, k_pool, v_pool, seq_lens, out, B, Hq, Hkv, D, scale);
    if (s != GQA_OK) return s;
    if (kv.type == kKvFp8 && D < 64) return GQA_ERR_UNSUPPORTED;  // E4M3: head_dim 64, 128 or 256
    if ((s = check_queries(B, M, Hq, Hkv, D)) != GQA_OK) return s;
    if (!isfinite(kv.k_scale) || !isfinite(kv.v_scale)) return GQA_ERR_SHAPE;
    if (B == 0) return (page_size > 0 && page_size % 16 == 0) ? GQA_OK : GQA_ERR_UNSUPPORTED;
    if (page_table == nullptr) return GQA_ERR_NULL;
    if (misaligned(page_table, 4)) return GQA_ERR_ALIGN;
    if (page_size <= 0 || num_pages <= 0 || max_pages <= 0 || num_splits < 0) return GQA_ERR_SHAPE;
    if (page_size % 16 != 0) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)max_pages * page_size > INT32_MAX || (int64_t)page_size * D * 2 > INT32_MAX)  // 32-bit offsets
        return GQA_ERR_SHAPE;
    if (workspace != nullptr && misaligned(workspace, 16)) return GQA_ERR_ALIGN;
    const gqa_tuning_t t = current_tuning();
    gqa_plan_t plan;
    s = plan_for_call(B, M * Hq, Hkv, D, max_pages * page_size, page_size, num_splits, t, &plan,
                      kv.type == kKvFp8 ? 1 : 2);
    if (s != GQA_OK) return s;
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return workspace == nullptr ? GQA_ERR_NULL : GQA_ERR_WORKSPACE;
    if (B == 0) return GQA_OK;
    SplitArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const unsigned char *>(k_pool);
    a.v = static_cast<const unsigned char *>(v_pool);
    a.seq_lens = seq_lens;
    a.page_table = page_table;
    a.out = out;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.M = M; a.R = M * (Hq / Hkv); a.qdiv = (256 + a.G - 1) / a.G;
    a.page_size = page_size;
    a.page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz((unsigned)page_size) : -1;
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    a.num_splits = plan.num_splits;
    a.split_tokens = plan.split_tokens;
    a.qk_scale_log2 = scale * kv.k_scale * 1.4426950408889634f;
    a.v_scale = kv.v_scale;
    return run(plan, t, a, D, true, kv.type, workspace, stream, phases);
}

}  // namespace

extern "C" {

gqa_status_t gqa_decode(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int S_max,
                        float scale, float *out, void *workspace, size_t workspace_bytes,
                        int num_splits, hipStream_t stream) {
    return decode_contig(q, k_cache, v_cache, seq_lens, B, 1, Hq, Hkv, D, S_max, scale, kBf16Cache, out,
                         workspace, workspace_bytes, num_splits, stream, kPhaseSplit | kPhaseCombine);
}

gqa_status_t gqa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int S_max,
                                 float scale, float *out, void *workspace, size_t workspace_bytes,
                                 int num_splits, hipStream_t stream) {
    return decode_contig(q, k_cache, v_cache, seq_lens, B, 1, Hq, Hkv, D, S_max, scale, kBf16Cache, out,
                         workspace, workspace_bytes, num_splits, stream, kPhaseSplit);
}

gqa_status_t gqa_paged_decode(const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *seq_lens, const int32_t *page_table, int B, int Hq,
                              int Hkv, int D, int page_size, int num_pages, int max_pages,
                              float scale, float *out, void *workspace, size_t workspace_bytes,
                              int num_splits, hipStream_t stream) {
    return decode_paged(q, k_pool, v_pool, seq_lens, page_table, B, 1, Hq, Hkv, D, page_size, num_pages,
                        max_pages, scale, kBf16Cache, out, workspace, workspace_bytes, num_splits,
                        stream, kPhaseSplit | kPhaseCombine);
}

gqa_status_t gqa_paged_decode_partials(const void *q, const void *k_pool, const void *v_pool,
                                       const int32_t *seq_lens, const int32_t *page_table, int B,
                                       int Hq, int Hkv, int D, int page_size, int num_pages,
                                       int max_pages, float scale, float *out, void *workspace,
                                       size_t workspace_bytes, int num_splits, hipStream_t stream) {
    return decode_paged(q, k_pool, v_pool, seq_lens, page_table, B, 1, Hq, Hkv, D, page_size, num_pages,
                        max_pages, scale, kBf16Cache, out, workspace, workspace_bytes, num_splits,
                        stream, kPhaseSplit);
}

gqa_status_t gqa_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int S_max,
                            float scale, float k_scale, float v_scale, float *out, void *workspace,
                            size_t workspace_bytes, int num_splits, hipStream_t stream) {
    return decode_contig(q, k_cache, v_cache, seq_lens, B, 1, Hq, Hkv, D, S_max, scale,
                         KvSpec{kKvFp8, k_scale, v_scale}, out, workspace, workspace_bytes, num_splits,
                         stream, kPhaseSplit | kPhaseCombine);
}

gqa_status_t gqa_paged_decode_fp8(const void *q, const void *k_pool, const void *v_pool,
                                  const int32_t *seq_lens, const int32_t *page_table, int B, int Hq,
                                  int Hkv, int D, int page_size, int num_pages, int max_pages,
                                  float scale, float k_scale, float v_scale, float *out,
                                  void *workspace, size_t workspace_bytes, int num_splits,
                                  hipStream_t stream) {
    return decode_paged(q, k_pool, v_pool, seq_lens, page_table, B, 1, Hq, Hkv, D, page_size, num_pages,
                        max_pages, scale, KvSpec{kKvFp8, k_scale, v_scale}, out, workspace,
                        workspace_bytes, num_splits, stream, kPhaseSplit | kPhaseCombine);
}

gqa_status_t gqa_decode_fp8_partials(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *seq_lens, int B, int Hq, int Hkv, int D,
                                     int S_max, float scale, float k_scale, float v_scale, float *out,
                                     void *workspace, size_t workspace_bytes, int num_splits,
                                     hipStream_t stream) {
    return decode_contig(q, k_cache, v_cache, seq_lens, B, 1, Hq, Hkv, D, S_max, scale,
                         KvSpec{kKvFp8, k_scale, v_scale}, out, workspace, workspace_bytes, num_splits,
                         stream, kPhaseSplit);
}

gqa_status_t gqa_paged_decode_fp8_partials(const void *q, const void *k_pool, const void *v_pool,
                                           const int32_t *seq_lens, const int32_t *page_table, int B,
                                           int Hq, int Hkv, int D, int page_size, int num_pages,
                                           int max_pages, float scale, float k_scale, float v_scale,
                                           float *out, void *workspace, size_t workspace_bytes,
                                           int num_splits, hipStream_t stream) {
    return decode_paged(q, k_pool, v_pool, seq_lens, page_table, B, 1, Hq, Hkv, D, page_size, num_pages,
                        max_pages, scale, KvSpec{kKvFp8, k_scale, v_scale}, out, workspace,
                        workspace_bytes, num_splits, stream, kPhaseSplit);
}

gqa_status_t gqa_decode_mq(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, int B, int M, int Hq, int Hkv, int D, int S_max,
                           float scale, float *out, void *workspace, size_t workspace_bytes,
                           int num_splits, hipStream_t stream) {
    return decode_contig(q, k_cache, v_cache, seq_lens, B, M, Hq, Hkv, D, S_max, scale, kBf16Cache, out,
                         workspace, workspace_bytes, num_splits, stream, kPhaseSplit | kPhaseCombine);
}

gqa_status_t gqa_paged_decode_mq(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *seq_lens, const int32_t *page_table, int B, int M,
                                 int Hq, int Hkv, int D, int page_size, int num_pages, int max_pages,
                                 float scale, float *out, void *workspace, size_t workspace_bytes,
                                 int num_splits, hipStream_t stream) {
    return decode_paged(q, k_pool, v_pool, seq_lens, page_table, B, M, Hq, Hkv, D, page_size, num_pages,
                        max_pages, scale, kBf16Cache, out, workspace, workspace_bytes, num_splits,
                        stream, kPhaseSplit | kPhaseCombine);
}

}  // extern "C"

namespace {

// ------------------------------------------------- the allocation-free call
//
// gqa_decode_noalloc keeps its partials (and the in-kernel fold's counters) in
// this file-scope device array instead of a caller's workspace.  In host code
// the name stands for a host-side shadow, not for device memory: the array's
// device address on each GPU comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is ever passed on.
constexpr size_t kScratchBytes = 4u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The arrival counters must start at zero (every call leaves them zero
// again): cleared once per device, by a kernel on the first call's stream
// (capturable; a clear that is replayed is harmless between calls).
__global__ void clear_counters_kernel(unsigned *counters) {
    for (int i = threadIdx.x; i < kMaxCounters; i += blockDim.x) counters[i] = 0u;
}

gqa_status_t scratch_for_device(hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GQA_ERR_HIP;
        if (launch(clear_counters_kernel, dim3(1), dim3(256), stream, static_cast<unsigned *>(ptr)) != hipSuccess)
            return GQA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status_t gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int S_max,
                                float scale, float *out, int num_splits, hipStream_t stream) {
    // The plan first, so that a call past the array's size is refused before
    // anything touches the device.
    gqa_status_t s = check_common(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, scale);
    if (s != GQA_OK || B == 0) return s;
    if (S_max < 0 || num_splits < 0) return GQA_ERR_SHAPE;
    gqa_plan_t plan;
    if ((s = plan_for_call(B, Hq, Hkv, D, S_max, 0, num_splits, current_tuning(), &plan)) != GQA_OK) return s;
    if (plan.workspace_bytes > kScratchBytes) return GQA_ERR_TOO_LARGE;
    void *ws = nullptr;
    if ((s = scratch_for_device(stream, &ws)) != GQA_OK) return s;
    return decode_contig(q, k_cache, v_cache, seq_lens, B, 1, Hq, Hkv, D, S_max, scale, kBf16Cache, out, ws,
                         kScratchBytes, num_splits, stream, kPhaseSplit | kPhaseCombine);
}

}  // extern "C"

namespace {

gqa_status_t combine_impl(const void *workspace, size_t workspace_bytes, const int32_t *seq_lens, int B, int Hq,
                          int Hkv, int D, int max_seq_len, int page_size, int num_splits, float *out,
                          hipStream_t stream, int elem_bytes) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_seq_len < 0 || page_size < 0 ||
        num_splits < 0)
        return GQA_ERR_SHAPE;
    if (!supported_dim(D) || Hq / Hkv > kMaxHeadsPerKv) return GQA_ERR_UNSUPPORTED;
    if (page_size > 0 && page_size % 16 != 0) return GQA_ERR_UNSUPPORTED;
    if (B == 0) return GQA_OK;
    if (out == nullptr || seq_lens == nullptr) return GQA_ERR_NULL;
    if (misaligned(out, 16) || misaligned(seq_lens, 4) ||
        (workspace != nullptr && misaligned(workspace, 16)))
        return GQA_ERR_ALIGN;
    const gqa_tuning_t t = current_tuning();
    gqa_plan_t plan;
    gqa_status_t s = plan_for_call(B, Hq, Hkv, D, max_seq_len, page_size, num_splits, t, &plan, elem_bytes);
    if (s != GQA_OK) return s;
    if (plan.direct) return GQA_OK;  // the split kernel already wrote `out`
    if (workspace == nullptr) return GQA_ERR_NULL;
    if (workspace_bytes < plan.workspace_bytes) return GQA_ERR_WORKSPACE;
    SplitArgs a{};
    a.out = out;
    a.seq_lens = seq_lens;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.M = 1; a.R = Hq / Hkv; a.qdiv = (256 + a.G - 1) / a.G;
    if (page_size > 0) {
        a.page_size = page_size;
        a.max_pages = max_seq_len / page_size;
    } else {
        a.S_max = max_seq_len;
    }
    // the cache type only matters for the share rule the split call used
    return run(plan, t, a, D, page_size > 0, elem_bytes == 1 ? kKvFp8 : kKvBf16, const_cast<void *>(workspace),
               stream, kPhaseCombine);
}

}  // namespace

extern "C" {

gqa_status_t gqa_decode_combine(const void *workspace, size_t workspace_bytes, const int32_t *seq_lens,
                                int B, int Hq, int Hkv, int D, int max_seq_len, int page_size,
                                int num_splits, float *out, hipStream_t stream) {
    return combine_impl(workspace, workspace_bytes, seq_lens, B, Hq, Hkv, D, max_seq_len, page_size, num_splits,
                        out, stream, 2);
}

gqa_status_t gqa_decode_combine_fp8(const void *workspace, size_t workspace_bytes, const int32_t *seq_lens,
                                    int B, int Hq, int Hkv, int D, int max_seq_len, int page_size,
                                    int num_splits, float *out, hipStream_t stream) {
    return combine_impl(workspace, workspace_bytes, seq_lens, B, Hq, Hkv, D, max_seq_len, page_size, num_splits,
                        out, stream, 1);
}

const char *gqa_status_string(gqa_status_t status) {
    // A C caller may pass any int: read it as one (an enum object holding a
    // value outside the enumerators must not be loaded as the enum in C++).
    static_assert(sizeof(gqa_status_t) == sizeof(int), "the C ABI passes the status as an int");
    int code;
    memcpy(&code, &status, sizeof code);
    switch (code) {
        case GQA_OK: return "ok";
        case GQA_ERR_NULL: return "a required pointer is NULL";
        case GQA_ERR_SHAPE: return "a size is out of range or inconsistent";
        case GQA_ERR_UNSUPPORTED: return "unsupported head_dim, group size or page size";
        case GQA_ERR_ALIGN: return "a pointer is not aligned as required";
        case GQA_ERR_WORKSPACE: return "workspace smaller than the plan needs";
        case GQA_ERR_HIP: return "a HIP runtime call or launch failed";
        case GQA_ERR_TOO_LARGE: return "the call needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

}  // extern "C"
