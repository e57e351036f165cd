// Weight gradient of the submanifold convolution for gfx950.
//
// The forward (page "mlx_backend/sparse_conv_metal.py", module docstring
// formula) is linear in w; its derivative contracted with dout is
//
//   dw[k, ci, co] = sum over n with nbr[k, n] present of feats[nbr[k, n], ci] * dout[n, co]
//
// i.e. for each offset k a GEMM featsᵀ·dout whose reduction runs over the N
// rows.  The reduction is split: workgroup (c, k, tile) sums rows of chunk c of
// the schedule (Morton order, 256-row tiles) into a TI x TO output tile held in
// MFMA accumulators, and writes it as an fp32 partial; a second kernel adds the
// chunks' partials in a fixed order, so the result does not depend on timing.
//
// Per 64-row unit the workgroup stages the gathered feats rows
// (feats[nbr[k, row]], zero where the neighbour is missing) and the dout rows
// (dout[order[row]], zero on padding rows) in LDS, row-major; 16-row blocks
// with no present neighbour at offset k are neither loaded nor multiplied.
// The chunk's units with any present neighbour at k are first compacted into
// an LDS list; the loop then runs over that list only, with each unit's rows
// loaded into registers WD units ahead and its neighbour indices 2*WD units
// further ahead, so that the dependent index -> row loads are in flight for
// several units' worth of MFMAs.
// Both MFMA operands have the rows as their reduction axis, so they are read
// column-wise: bf16 fragments with the transposing ds_read_b64_tr_b16, fp32
// fragments with one 4-byte read per lane.  Row pitches are padded so that
// those reads are free of bank conflicts over each half-wave (128 banks).
#include "spconv_internal.h"

#include <algorithm>
#include <type_traits>

namespace spc {

namespace {

typedef uint32_t u32x4w_t __attribute__((ext_vector_type(4)));
typedef float f32x4w_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4w_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8w_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) bf16x4w_t lds_bf16x4w_t;

struct WgradParams {
    const void* feats;
    const void* dout;
    const int32_t* nbr_m;
    const int32_t* order;
    const uint16_t* blkmask;
    float* part;
    int64_t N, Npad;
    int K, Ci, Co;
    int nchunks, units_per_chunk;
};

constexpr int kWgThreads = 512;   // 8 waves

// wave layout over the TI x TO output tile: WB waves own RB x CB 16x16 blocks
// each, WK waves share a block set and split the k-steps.  SPLIT: four waves
// per block set and two sets taking alternate k-steps, so that each wave's
// block set is twice as large and its fragment reads per MFMA fall by a third
// (surf1024 15.6 -> 12.5 ms, surf512d2 12.1 -> 8.4 ms); fp32 at 128 x 128
// keeps eight sets (the larger set spills)
template <int TI, int TO, bool SPLIT>
struct WgShape {
    static constexpr int NBI = TI / 16, NBO = TO / 16, NBLK = NBI * NBO;
    static constexpr int BPW = NBLK >= 8 ? (SPLIT ? NBLK / 4 : NBLK / 8) : 1;
    static constexpr int RB = BPW == 16 ? 4 : (BPW == 8 ? 4 : (BPW == 4 ? 2 : (BPW == 2 ? (NBI >= 2 * NBO ? 2 : (NBO >= 2 * NBI ? 1 : 2)) : 1)));
    static constexpr int CB = BPW / RB;
    static constexpr int WB = NBLK / BPW;
    static constexpr int WK = 8 / WB;
    static_assert(RB * CB == BPW && NBI % RB == 0 && NBO % CB == 0, "wave blocks tile the output");
    static_assert((NBI / RB) * (NBO / CB) == WB && WB * WK == 8, "8 waves");
};

// LDS row pitch in bytes for rows of C channels of ES-byte elements
template <int C, int ES>
constexpr int wg_pitch() {
    return ES == 2 ? (C == 32 ? 80 : (C == 64 ? 160 : 272)) : C * 4 + 64;
}

// Rows per staged unit: 64 (bf16 and fp32).
constexpr int wg_rows(bool) { return 64; }

// fp32 stage pitch in 4-byte words for rows of C channels read W consecutive
// channels per lane by the four lane groups (rows 4q + g): W = 1, C + 16
// (16-word windows at distinct banks); W = 2, the smallest P >= C with
// P = 32 or 96 mod 128 (four 32-word windows tile the 128 banks); W = 4, the
// smallest P >= C with P = 64 mod 128 (each half-wave's two 64-word windows)
constexpr int wg_pitch32(int C, int W) {
    if (W == 1) return C + 16;
    int P = C;
    while (W == 2 ? (P % 128 != 32 && P % 128 != 96) : P % 128 != 64) ++P;
    return P;
}
// Units whose rows are in flight (register stages; fp32 rows take twice the
// registers) and index look-ahead.
constexpr int wg_data_stages(bool bf16) { return bf16 ? 3 : 2; }

// f(integral_constant<J>, i0 + J) for J = 0 .. W-1 while i0 + J < n; false
// once the list ends
template <int J, int W, typename F>
__device__ __forceinline__ bool wg_steps(F& f, int i0, int n) {
    if constexpr (J == W) {
        return true;
    } else {
        if (i0 + J >= n) return false;
        f(std::integral_constant<int, J>{}, i0 + J);
        return wg_steps<J + 1, W>(f, i0, n);
    }
}
// Active units compacted per batch (LDS list entries).
constexpr int kWgUnitBatch = 2048;

// W consecutive floats of a stage row (W = 1, 2 or 4; 4 W-byte aligned)
template <int W>
__device__ __forceinline__ void wg_read_vec(const uint8_t* p, float (&v)[W]) {
    if constexpr (W == 4) {
        const f32x4w_t x = *(const f32x4w_t*)p;
        v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    } else if constexpr (W == 2) {
        const float2 x = *(const float2*)p;
        v[0] = x.x; v[1] = x.y;
    } else {
        v[0] = *(const float*)p;
    }
}

template <bool BF16, int TI, int TO>
__global__ void __launch_bounds__(kWgThreads) k_wgrad(WgradParams p) {
    using S = WgShape<TI, TO, BF16 || TI * TO < 128 * 128>;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int UR = wg_rows(BF16);                 // rows per unit
    // fp32: lane a takes input channels 16 bi0 + RB a + i and output channels
    // 16 bo0 + CB a + j (VEC), so its operands of all its blocks are one read
    // of RB (CB) consecutive floats, where the stages with the pitches that
    // keep those reads free of bank conflicts fit the LDS; else one channel
    // per block (16 blk + a)
    constexpr bool VEC = !BF16 && 2 * UR * 4 * (wg_pitch32(TI, S::RB) + wg_pitch32(TO, S::CB)) +
                                          4 * kWgUnitBatch + 64 <= 160 * 1024;
    constexpr int FP = VEC ? 4 * wg_pitch32(TI, S::RB) : wg_pitch<TI, ES>();
    constexpr int DP = VEC ? 4 * wg_pitch32(TO, S::CB) : wg_pitch<TO, ES>();
    constexpr int SF = TI * ES / 16, SD = TO * ES / 16; // 16-byte segments per row
    constexpr int NF = UR * SF, ND = UR * SD;         // 16-byte segments per unit
    constexpr int NFL = (NF + kWgThreads - 1) / kWgThreads, NDL = (ND + kWgThreads - 1) / kWgThreads;
    constexpr int KS = UR / 32;                       // 32-row k-steps per unit
    static_assert(2 * UR * (FP + DP) <= 160 * 1024, "stages fit the LDS");

    // two feats stages, two dout stages; after the loop the same bytes hold
    // the k-split waves' partial tiles for the final sum
    constexpr int STAGE_BYTES = 2 * UR * (FP + DP);
    constexpr int RED_BYTES = (S::WK - 1) * S::NBLK * 256 * 4;
    static_assert(RED_BYTES <= STAGE_BYTES, "the k-split partials fit in the stages");
    __shared__ __attribute__((aligned(16))) uint8_t stg[STAGE_BYTES];
    auto fst = [&](int b) -> uint8_t* { return stg + b * (UR * FP); };
    auto dstg = [&](int b) -> uint8_t* { return stg + 2 * UR * FP + b * (UR * DP); };
    __shared__ uint32_t ulist[kWgUnitBatch];   // (unit - batch base) | block mask << 16
    __shared__ int wcnt[kWgThreads / 64];

    const int t = threadIdx.x, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wb = wv % S::WB, wk = wv / S::WB;
    const int bi0 = (wb / (S::NBO / S::CB)) * S::RB, bo0 = (wb % (S::NBO / S::CB)) * S::CB;
    const int c = blockIdx.x, k = blockIdx.y;
    const int nto = p.Co / TO;
    const int ti = blockIdx.z / nto, to = blockIdx.z % nto;
    const int ci0 = ti * TI, co0 = to * TO;
    const int64_t nunits = p.Npad / UR;
    const int64_t u0 = (int64_t)c * p.units_per_chunk;
    const int64_t u1 = u0 + p.units_per_chunk < nunits ? u0 + p.units_per_chunk : nunits;
    const uint32_t N32 = (uint32_t)p.N;
    const uint8_t* feats = (const uint8_t*)p.feats;
    const uint8_t* dout = (const uint8_t*)p.dout;

    f32x4w_t acc[S::RB][S::CB];
#pragma unroll
    for (int i = 0; i < S::RB; ++i)
#pragma unroll
        for (int j = 0; j < S::CB; ++j) acc[i][j] = f32x4w_t{0.f, 0.f, 0.f, 0.f};

    // active 16-row blocks of unit u at offset k (bit b = rows 16b .. 16b+15)
    auto unit_mask = [&](int64_t u) -> uint32_t {
        const int64_t r0 = u * UR;
        return (uint32_t)(p.blkmask[(r0 / kTileRows) * p.K + k] >> (int)((r0 % kTileRows) / 16)) &
               ((1u << (UR / 16)) - 1u);
    };
    // per-thread source rows of a unit: feats row (caller index of the
    // neighbour, or N) and dout row (caller index, or -1)
    struct Idx {
        uint32_t f[NFL];
        int32_t d[NDL];
    };
    // list entry e (mask 0: nothing is loaded) of the batch starting at unit ub
    auto load_idx = [&](int64_t ub, uint32_t ent, Idx& x) {
        const uint32_t m = ent >> 16;
        const int64_t r0 = (ub + (int64_t)(ent & 0xFFFFu)) * UR;
#pragma unroll
        for (int i = 0; i < NFL; ++i) {
            const int e = t + kWgThreads * i, row = e / SF;
            x.f[i] = (e < NF && ((m >> (row / 16)) & 1u)) ? (uint32_t)p.nbr_m[(int64_t)k * p.Npad + r0 + row] : N32;
        }
#pragma unroll
        for (int i = 0; i < NDL; ++i) {
            const int e = t + kWgThreads * i, row = e / SD;
            x.d[i] = (e < ND && ((m >> (row / 16)) & 1u)) ? p.order[r0 + row] : -1;
        }
    };
    struct Dat {
        u32x4w_t f[NFL], d[NDL];
    };
    auto load_dat = [&](const Idx& x, Dat& v) {
#pragma unroll
        for (int i = 0; i < NFL; ++i) {
            const int seg = (t + kWgThreads * i) % SF;
            v.f[i] = u32x4w_t{0u, 0u, 0u, 0u};
            if (x.f[i] < N32) v.f[i] = *(const u32x4w_t*)(feats + ((int64_t)x.f[i] * p.Ci + ci0) * ES + 16 * seg);
        }
#pragma unroll
        for (int i = 0; i < NDL; ++i) {
            const int seg = (t + kWgThreads * i) % SD;
            v.d[i] = u32x4w_t{0u, 0u, 0u, 0u};
            if (x.d[i] >= 0) v.d[i] = *(const u32x4w_t*)(dout + ((int64_t)x.d[i] * p.Co + co0) * ES + 16 * seg);
        }
    };
    auto store_dat = [&](const Dat& v, int b) {
#pragma unroll
        for (int i = 0; i < NFL; ++i) {
            const int e = t + kWgThreads * i;
            if (e < NF) *(u32x4w_t*)(fst(b) + (e / SF) * FP + 16 * (e % SF)) = v.f[i];
        }
#pragma unroll
        for (int i = 0; i < NDL; ++i) {
            const int e = t + kWgThreads * i;
            if (e < ND) *(u32x4w_t*)(dstg(b) + (e / SD) * DP + 16 * (e % SD)) = v.d[i];
        }
    };

    const int g = lane >> 4, a = lane & 15;
    // MFMAs over the staged unit in buffer b
    auto compute = [&](int b, uint32_t m) {
        const uint8_t* fs = fst(b);
        const uint8_t* ds = dstg(b);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s % S::WK != wk || !((m >> (2 * s)) & 3u)) continue;
            if constexpr (BF16) {
                // lane a of group g addresses row 32s + 8g + 4h + a/4, channel
                // 16*blk + 4*(a%4); the transposing read hands lane a the four
                // rows' values of channel 16*blk + a
                bf16x8w_t af[S::RB], bf[S::CB];
#pragma unroll
                for (int i = 0; i < S::RB; ++i) {
                    const int col = 16 * (bi0 + i) + 4 * (a & 3);
                    bf16x4w_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4w_t*)(fs + (32 * s + 8 * g + (a >> 2)) * FP + 2 * col));
                    bf16x4w_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4w_t*)(fs + (32 * s + 8 * g + 4 + (a >> 2)) * FP + 2 * col));
                    af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int j = 0; j < S::CB; ++j) {
                    const int col = 16 * (bo0 + j) + 4 * (a & 3);
                    bf16x4w_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4w_t*)(ds + (32 * s + 8 * g + (a >> 2)) * DP + 2 * col));
                    bf16x4w_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4w_t*)(ds + (32 * s + 8 * g + 4 + (a >> 2)) * DP + 2 * col));
                    bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int i = 0; i < S::RB; ++i)
#pragma unroll
                    for (int j = 0; j < S::CB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
            } else {
                // four rows per MFMA: lane (a, g) reads row 32s + 4q + g
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int row = 32 * s + 4 * q + g;
                    float af[S::RB], bf[S::CB];
                    if constexpr (VEC) {
                        wg_read_vec<S::RB>(fs + row * FP + 4 * (16 * bi0 + S::RB * a), af);
                        wg_read_vec<S::CB>(ds + row * DP + 4 * (16 * bo0 + S::CB * a), bf);
                    } else {
#pragma unroll
                        for (int i = 0; i < S::RB; ++i) af[i] = *(const float*)(fs + row * FP + 4 * (16 * (bi0 + i) + a));
#pragma unroll
                        for (int j = 0; j < S::CB; ++j) bf[j] = *(const float*)(ds + row * DP + 4 * (16 * (bo0 + j) + a));
                    }
#pragma unroll
                    for (int i = 0; i < S::RB; ++i)
#pragma unroll
                        for (int j = 0; j < S::CB; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bf[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    // Batches of the chunk's units: compact the active ones into ulist, then
    // run the pipeline over the list.  Stage indices are compile-time (the
    // loop body is unrolled over the index ring), so the ring lives in VGPRs.
    constexpr int WD = wg_data_stages(BF16), WI = 2 * WD;
    int buf = 0;
    for (int64_t ub = u0; ub < u1; ub += kWgUnitBatch) {
        const int64_t ue = ub + kWgUnitBatch < u1 ? ub + kWgUnitBatch : u1;
        int n = 0;
        for (int64_t s0 = ub; s0 < ue; s0 += kWgThreads) {
            const int64_t u = s0 + t;
            const uint32_t m = u < ue ? unit_mask(u) : 0u;
            const uint64_t bal = __ballot(m != 0u);
            const int rank = __popcll(bal & ((1ull << lane) - 1ull));
            if (lane == 0) wcnt[wv] = __popcll(bal);
            __syncthreads();
            int off = n, tot = n;
#pragma unroll
            for (int v = 0; v < kWgThreads / 64; ++v) {
                off += v < wv ? wcnt[v] : 0;
                tot += wcnt[v];
            }
            if (m) ulist[off + rank] = (uint32_t)(u - ub) | (m << 16);
            n = tot;
            __syncthreads();
        }
        auto entry = [&](int i) -> uint32_t {
            return i < n ? (uint32_t)__builtin_amdgcn_readfirstlane((int)ulist[i]) : 0u;
        };
        Idx xs[WI];
        Dat ds[WD];
#pragma unroll
        for (int j = 0; j < WI; ++j) load_idx(ub, entry(j), xs[j]);
#pragma unroll
        for (int j = 0; j < WD - 1; ++j) {
            load_dat(xs[j], ds[j]);
            load_idx(ub, entry(j + WI), xs[j]);
        }
        // iteration i: rows of entry i + WD - 1 go out (their indices were
        // loaded WI iterations earlier), then the indices of entry
        // i + WD - 1 + WI take their stage; entry i is staged and multiplied
        auto step = [&](auto jc, int i) {
            constexpr int J = decltype(jc)::value;
            constexpr int SI = (J + WD - 1) % WI, SD = (J + WD - 1) % WD, SC = J % WD;
            load_dat(xs[SI], ds[SD]);
            load_idx(ub, entry(i + WD - 1 + WI), xs[SI]);
            const uint32_t m = entry(i) >> 16;
            store_dat(ds[SC], buf);
            // the stage is written before anyone reads it; the rows and
            // indices of later units stay in flight across the barrier
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            barrier_only();
            compute(buf, m);
            buf ^= 1;
        };
        for (int i0 = 0; i0 < n; i0 += WI)
            if (!wg_steps<0, WI>(step, i0, n)) break;
        __syncthreads();   // the list and the stages are reused by the next batch
    }

    // waves that split the k-steps of one block set add up through LDS
    float* red = (float*)stg;
    if constexpr (S::WK > 1) {
        __syncthreads();
        if (wk > 0) {
#pragma unroll
            for (int i = 0; i < S::RB; ++i)
#pragma unroll
                for (int j = 0; j < S::CB; ++j)
                    *(f32x4w_t*)(red + (((wk - 1) * S::WB + wb) * S::RB * S::CB + i * S::CB + j) * 256 + 4 * lane) =
                        acc[i][j];
        }
        __syncthreads();
        if (wk == 0) {
            for (int w2 = 1; w2 < S::WK; ++w2)
#pragma unroll
                for (int i = 0; i < S::RB; ++i)
#pragma unroll
                    for (int j = 0; j < S::CB; ++j)
                        acc[i][j] += *(const f32x4w_t*)(red + (((w2 - 1) * S::WB + wb) * S::RB * S::CB + i * S::CB + j) *
                                                                  256 + 4 * lane);
        }
    }
    if (wk == 0) {
        // lane (a, g) holds rows 4g .. 4g+3 (input channels), column a (output channel) of each block
        float* out = p.part + ((((int64_t)k * (p.Ci / TI) + ti) * nto + to) * p.nchunks + c) * (TI * TO);
#pragma unroll
        for (int i = 0; i < S::RB; ++i)
#pragma unroll
            for (int j = 0; j < S::CB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (VEC)
                        out[(16 * bi0 + S::RB * (4 * g + e) + i) * TO + 16 * bo0 + S::CB * a + j] = acc[i][j][e];
                    else
                        out[(16 * (bi0 + i) + 4 * g + e) * TO + 16 * (bo0 + j) + a] = acc[i][j][e];
                }
    }
}

// ---------------------------------------------------------------------------
// Grouped offsets (bf16, Ci tile 128, Co tile 64 or 128).  Workgroup (chunk c,
// offset group g, output tile) accumulates dw[k] for the kWgGroup offsets
// k = g*kWgGroup ... at once.  Each unit's dout rows are gathered and staged
// once for all of them, and each wave's dout fragments feed the MFMAs of every
// offset of the group; the feats gathers of the group (neighbours of the same
// rows one z-step apart) share L2 lines.  Per unit, 16-row blocks with no
// present neighbour at an offset are neither loaded nor multiplied for it.
// Rows go into registers one unit ahead and indices two, as in k_wgrad.
// ---------------------------------------------------------------------------
constexpr int kWgGroup = 3;

template <int TI, int TO>
struct WgGShape {   // 8 waves of RB x CB 16x16 blocks each
    static constexpr int NBI = TI / 16, NBO = TO / 16;
    static constexpr int RB = 2, CB = NBI * NBO / (8 * RB);
    static_assert(CB >= 1 && NBO % CB == 0 && (NBI / RB) * (NBO / CB) == 8, "eight waves tile the output");
};

template <int TI, int TO>
__global__ void __launch_bounds__(kWgThreads) k_wgrad_g(WgradParams p) {
    constexpr int KG = kWgGroup;
    using S = WgGShape<TI, TO>;
    constexpr int ES = 2, UR = 64;
    constexpr int FP = wg_pitch<TI, ES>(), DP = wg_pitch<TO, ES>();
    constexpr int SF = TI * ES / 16, SD = TO * ES / 16;   // 16-byte segments per row
    constexpr int NF = UR * SF, ND = UR * SD;             // 16-byte segments per unit
    static_assert(NF % kWgThreads == 0 && ND % kWgThreads == 0, "whole segments per thread");
    constexpr int NFL = NF / kWgThreads, NDL = ND / kWgThreads;
    constexpr int KS = UR / 32;                           // 32-row k-steps per unit
    constexpr int FST = UR * FP, DST = UR * DP;           // one feats / dout stage
    constexpr int BUF = DST + KG * FST;                   // one buffer: dout + the group's feats
    static_assert(2 * BUF + 4 * kWgUnitBatch <= 160 * 1024, "stages fit the LDS");
    static_assert(4 * KG + 11 <= 32 && kWgUnitBatch <= 2048, "list entry: 11-bit unit, 4-bit masks");
    constexpr int WD = 2, WI = 2;                         // units of rows / indices in flight

    __shared__ __attribute__((aligned(16))) uint8_t stg[2 * BUF];
    __shared__ uint32_t ulist[kWgUnitBatch];              // (unit - batch base) | mask(kg) << (11 + 4 kg)
    __shared__ int wcnt[kWgThreads / 64];

    const int t = threadIdx.x, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int bi0 = (wv % (S::NBI / S::RB)) * S::RB, bo0 = (wv / (S::NBI / S::RB)) * S::CB;
    // (chunk, offset group, output tile) from the one-dimensional grid: the
    // workgroups of one chunk are consecutive on one XCD (workgroup b runs on
    // XCD b % 8), so that the chunk's dout rows and neighbour rows, read by
    // every group and tile, are fetched into that XCD's L2 about once
    const int ngr = (p.K + KG - 1) / KG;
    const int nto = p.Co / TO;
    const int per_chunk = ngr * (p.Ci / TI) * nto;
    int c, r;
    if (p.nchunks % 8 == 0) {
        const int b = (int)blockIdx.x, x = b & 7, l = b >> 3;
        c = x + 8 * (l / per_chunk);
        r = l % per_chunk;
    } else {
        c = (int)blockIdx.x / per_chunk;
        r = (int)blockIdx.x % per_chunk;
    }
    const int k0 = (r % ngr) * KG;
    const int kn = p.K - k0 < KG ? p.K - k0 : KG;         // offsets of this group
    const int ti = (r / ngr) / nto, to = (r / ngr) % nto;
    const int ci0 = ti * TI, co0 = to * TO;
    const int64_t nunits = p.Npad / UR;
    const int64_t u0 = (int64_t)c * p.units_per_chunk;
    const int64_t u1 = u0 + p.units_per_chunk < nunits ? u0 + p.units_per_chunk : nunits;
    const uint32_t N32 = (uint32_t)p.N;
    const uint8_t* feats = (const uint8_t*)p.feats;
    const uint8_t* dout = (const uint8_t*)p.dout;

    f32x4w_t acc[KG][S::RB][S::CB];
#pragma unroll
    for (int g = 0; g < KG; ++g)
#pragma unroll
        for (int i = 0; i < S::RB; ++i)
#pragma unroll
            for (int j = 0; j < S::CB; ++j) acc[g][i][j] = f32x4w_t{0.f, 0.f, 0.f, 0.f};

    auto emask = [](uint32_t ent, int g) -> uint32_t { return (ent >> (11 + 4 * g)) & 0xFu; };
    struct Idx {
        uint32_t f[KG][NFL];
        int32_t d[NDL];
    };
    auto load_idx = [&](int64_t ub, uint32_t ent, Idx& x) {
        const int64_t r0 = (ub + (int64_t)(ent & 0x7FFu)) * UR;
        uint32_t many = 0;
#pragma unroll
        for (int g = 0; g < KG; ++g) many |= emask(ent, g);
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            const uint32_t m = emask(ent, g);
#pragma unroll
            for (int i = 0; i < NFL; ++i) {
                const int row = (t + kWgThreads * i) / SF;
                x.f[g][i] = ((m >> (row / 16)) & 1u) ? (uint32_t)p.nbr_m[(int64_t)(k0 + g) * p.Npad + r0 + row] : N32;
            }
        }
#pragma unroll
        for (int i = 0; i < NDL; ++i) {
            const int row = (t + kWgThreads * i) / SD;
            x.d[i] = ((many >> (row / 16)) & 1u) ? p.order[r0 + row] : -1;
        }
    };
    struct Dat {
        u32x4w_t f[KG][NFL], d[NDL];
    };
    auto load_dat = [&](const Idx& x, Dat& v) {
#pragma unroll
        for (int g = 0; g < KG; ++g)
#pragma unroll
            for (int i = 0; i < NFL; ++i) {
                const int seg = (t + kWgThreads * i) % SF;
                v.f[g][i] = u32x4w_t{0u, 0u, 0u, 0u};
                if (x.f[g][i] < N32)
                    v.f[g][i] = *(const u32x4w_t*)(feats + ((int64_t)x.f[g][i] * p.Ci + ci0) * ES + 16 * seg);
            }
#pragma unroll
        for (int i = 0; i < NDL; ++i) {
            const int seg = (t + kWgThreads * i) % SD;
            v.d[i] = u32x4w_t{0u, 0u, 0u, 0u};
            if (x.d[i] >= 0) v.d[i] = *(const u32x4w_t*)(dout + ((int64_t)x.d[i] * p.Co + co0) * ES + 16 * seg);
        }
    };
    auto store_dat = [&](const Dat& v, int b) {
        uint8_t* base = stg + b * BUF;
#pragma unroll
        for (int i = 0; i < NDL; ++i) {
            const int e = t + kWgThreads * i;
            *(u32x4w_t*)(base + (e / SD) * DP + 16 * (e % SD)) = v.d[i];
        }
#pragma unroll
        for (int g = 0; g < KG; ++g)
#pragma unroll
            for (int i = 0; i < NFL; ++i) {
                const int e = t + kWgThreads * i;
                *(u32x4w_t*)(base + DST + g * FST + (e / SF) * FP + 16 * (e % SF)) = v.f[g][i];
            }
    };

    const int g4 = lane >> 4, a = lane & 15;
    // transposed fragment of 16 channels at channel 16*blk of a row-major stage:
    // lane a of group g4 addresses rows 32s + 8*g4 + 4h + a/4, channel 16*blk + 4*(a%4)
    auto frag = [&](const uint8_t* st, int pitch, int s, int blk) -> bf16x8w_t {
        const int col = 16 * blk + 4 * (a & 3);
        bf16x4w_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4w_t*)(st + (32 * s + 8 * g4 + (a >> 2)) * pitch + 2 * col));
        bf16x4w_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4w_t*)(st + (32 * s + 8 * g4 + 4 + (a >> 2)) * pitch + 2 * col));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto compute = [&](int b, uint32_t ent) {
        const uint8_t* base = stg + b * BUF;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint32_t any = 0;
#pragma unroll
            for (int g = 0; g < KG; ++g) any |= (emask(ent, g) >> (2 * s)) & 3u;
            if (!any) continue;
            bf16x8w_t bf[S::CB];
#pragma unroll
            for (int j = 0; j < S::CB; ++j) bf[j] = frag(base, DP, s, bo0 + j);
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                if (!((emask(ent, g) >> (2 * s)) & 3u)) continue;
                bf16x8w_t af[S::RB];
#pragma unroll
                for (int i = 0; i < S::RB; ++i) af[i] = frag(base + DST + g * FST, FP, s, bi0 + i);
#pragma unroll
                for (int i = 0; i < S::RB; ++i)
#pragma unroll
                    for (int j = 0; j < S::CB; ++j)
                        acc[g][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[g][i][j], 0, 0, 0);
            }
        }
    };

    int buf = 0;
    for (int64_t ub = u0; ub < u1; ub += kWgUnitBatch) {
        const int64_t ue = ub + kWgUnitBatch < u1 ? ub + kWgUnitBatch : u1;
        int n = 0;
        for (int64_t s0 = ub; s0 < ue; s0 += kWgThreads) {
            const int64_t u = s0 + t;
            uint32_t ms = 0;
            if (u < ue) {
                const int64_t r0 = u * UR;
                const int64_t mrow = (r0 / kTileRows) * p.K;
                const int sh = (int)((r0 % kTileRows) / 16);
#pragma unroll
                for (int g = 0; g < KG; ++g)
                    if (g < kn) ms |= (((uint32_t)p.blkmask[mrow + k0 + g] >> sh) & 0xFu) << (4 * g);
            }
            const uint64_t bal = __ballot(ms != 0u);
            const int rank = __popcll(bal & ((1ull << lane) - 1ull));
            if (lane == 0) wcnt[wv] = __popcll(bal);
            __syncthreads();
            int off = n, tot = n;
#pragma unroll
            for (int v = 0; v < kWgThreads / 64; ++v) {
                off += v < wv ? wcnt[v] : 0;
                tot += wcnt[v];
            }
            if (ms) ulist[off + rank] = (uint32_t)(u - ub) | (ms << 11);
            n = tot;
            __syncthreads();
        }
        auto entry = [&](int i) -> uint32_t {
            return i < n ? (uint32_t)__builtin_amdgcn_readfirstlane((int)ulist[i]) : 0u;
        };
        Idx xs[WI];
        Dat ds[WD];
#pragma unroll
        for (int j = 0; j < WI; ++j) load_idx(ub, entry(j), xs[j]);
#pragma unroll
        for (int j = 0; j < WD - 1; ++j) {
            load_dat(xs[j], ds[j]);
            load_idx(ub, entry(j + WI), xs[j]);
        }
        auto step = [&](auto jc, int i) {
            constexpr int J = decltype(jc)::value;
            constexpr int SI = (J + WD - 1) % WI, SD_ = (J + WD - 1) % WD, SC = J % WD;
            load_dat(xs[SI], ds[SD_]);
            load_idx(ub, entry(i + WD - 1 + WI), xs[SI]);
            const uint32_t ent = entry(i);
            store_dat(ds[SC], buf);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the stage is written
            barrier_only();
            compute(buf, ent);
            buf ^= 1;
        };
        for (int i0 = 0; i0 < n; i0 += WI)
            if (!wg_steps<0, WI>(step, i0, n)) break;
        __syncthreads();   // the list and the stages are reused by the next batch
    }

    // lane (a, g4) holds rows 4*g4 .. 4*g4+3 (input channels), column a (output channel) of each block
#pragma unroll
    for (int g = 0; g < KG; ++g) {
        if (g >= kn) break;
        float* out = p.part + ((((int64_t)(k0 + g) * (p.Ci / TI) + ti) * nto + to) * p.nchunks + c) * (TI * TO);
#pragma unroll
        for (int i = 0; i < S::RB; ++i)
#pragma unroll
            for (int j = 0; j < S::CB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[(16 * (bi0 + i) + 4 * g4 + e) * TO + 16 * (bo0 + j) + a] = acc[g][i][j][e];
    }
}

// ---------------------------------------------------------------------------
// Weight gradient over the map's distinct-row lists (bf16, K <= 27, Ci and Co
// multiples of 32, maps whose half tiles all have lists).  Workgroup (chunk c,
// slice (ti, to)) sums, over the half tiles of chunk c, the 27 x 32 x 32
// block dw[k][32 ti .. + 31][32 to .. + 31] of every offset: per half tile
// (128 schedule rows) it stages once
//   * the 32-channel slices of the half tile's distinct neighbour rows (slot s
//     of its list at 64 s; slot kDistinctCap stays zero: a missing neighbour),
//   * the 32-channel slices of its 128 dout rows (dout[order[row]], zero on
//     padding rows),
//   * the half tile's slot codes (K x 128 uint16),
// and every offset's MFMAs read the rows of its neighbours through the codes.
// A half tile with layered lists is staged once per layer (its offsets 9p ..
// 9p + 8 read that layer's list).  The four waves take the offsets k = wave +
// 4 i.  Staging is double-buffered: a unit's rows are loaded into registers
// during the previous unit's MFMAs and written to the other LDS buffer, so one
// barrier per unit separates the two.  Both MFMA operands have the rows as
// their reduction axis and are read with the transposing ds_read_b64_tr_b16;
// the 32-byte halves of a staged row are swapped on odd 8-row groups so that
// a half-wave's 8 rows fall on distinct banks (dout rows always; neighbour
// rows when their slots differ modulo 16).
// ---------------------------------------------------------------------------
constexpr int kWtThreads = 256;                        // 4 waves
constexpr int kWtMaxOff = (kDistinctMaxK + 3) / 4;     // offsets per wave
constexpr int kWtXRows = 320;                          // staged list slots (5 per thread)
constexpr int kWtDout = kWtXRows * 64;                 // byte offset of the dout rows
constexpr int kWtCodes = kWtDout + kDistinctRows * 64;
constexpr int kWtStage = kWtCodes + kDistinctMaxK * kDistinctRows * 2;
constexpr int kWtMaxHalves = 1024;                     // half tiles per chunk (their counts in LDS)
static_assert(kWtXRows > kDistinctCap && kWtXRows == 5 * kWtThreads / 4, "list slots");
static_assert(2 * kWtStage + 4 * kWtMaxHalves <= 80 * 1024, "two workgroups per CU");

struct WtParams {
    const uint8_t* feats;
    const uint8_t* dout;
    const int32_t* order;
    const uint16_t* blkmask;
    const uint32_t* dcount;
    const int32_t* drow;
    const uint16_t* smap;
    float* part;
    int64_t N;
    int K, Ci, Co;
    int nhalf, nchunks, per_chunk;   // half tiles, chunks, half tiles per chunk
};

__global__ void __launch_bounds__(kWtThreads, 2) k_wgrad_tile(WtParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t stg[2 * kWtStage];
    __shared__ uint32_t dcs[kWtMaxHalves];

    const int t = threadIdx.x, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int g4 = lane >> 4, a = lane & 15;
    const int K = p.K;
    const int nti = p.Ci / 32, nto = p.Co / 32, nsl = nti * nto;
    // (chunk, slice) from the one-dimensional grid: a chunk's slices are
    // consecutive on one XCD (workgroup b runs on XCD b % 8), so that the
    // chunk's rows come into that XCD's L2 about once
    int c, sl;
    if (p.nchunks % 8 == 0) {
        const int b = (int)blockIdx.x, x = b & 7, l = b >> 3;
        c = x + 8 * (l / nsl);
        sl = l % nsl;
    } else {
        c = (int)blockIdx.x / nsl;
        sl = (int)blockIdx.x % nsl;
    }
    const int ti = sl / nto, to = sl % nto;
    const int ci0 = 32 * ti, co0 = 32 * to;
    const int q0 = c * p.per_chunk;
    const int nq = max(min(q0 + p.per_chunk, p.nhalf) - q0, 0);   // half tiles of the chunk
    const uint32_t N32 = (uint32_t)p.N;

    for (int i = t; i < nq; i += kWtThreads) dcs[i] = p.dcount[q0 + i];
    // the zero row of both buffers
    if (t < 8) *(u32x4w_t*)(stg + (t >> 2) * kWtStage + kDistinctCap * 64 + 16 * (t & 3)) = u32x4w_t{0u, 0u, 0u, 0u};
    __syncthreads();

    // units: (half tile, pass), passes = 3 for layered lists
    auto npass = [&](int qi) -> int { return (dcs[qi] & kLayerPasses) ? kDistinctLayers : 1; };
    auto rows_of = [&](int qi, int ps) -> int {
        const uint32_t d = dcs[qi];
        const int n = (d & kLayerPasses) ? layer_rows(d, ps) : (int)d;
        return n < kDistinctCap ? n : kDistinctCap;   // (every slot below the zero row)
    };
    auto advance = [&](int& qi, int& ps) {
        if (++ps >= npass(qi)) {
            ++qi;
            ps = 0;
        }
    };

    f32x4w_t acc[kWtMaxOff][2][2];
#pragma unroll
    for (int i = 0; i < kWtMaxOff; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v) acc[i][u][v] = f32x4w_t{0.f, 0.f, 0.f, 0.f};

    // this thread's share of a unit: list slots (t >> 2) + 64 j (j < 5) and
    // dout rows (t >> 2) + 64 j (j < 2), 16-byte chunk t & 3 of each; 16-byte
    // pieces t and t + 256 of the slot codes
    const int tr = t >> 2, tc = t & 3;
    struct Idx {
        int32_t x[5], d[2];
        int dcp, qi;
    };
    struct Dat {
        u32x4w_t x[5], d[2], s[2];
    };
    auto load_idx = [&](int qi, int ps, Idx& ix) {
        ix.dcp = rows_of(qi, ps);
        ix.qi = qi;
        const int32_t* dr = p.drow + (int64_t)(q0 + qi) * kDistinctListCap + kDistinctCap * ps;
#pragma unroll
        for (int j = 0; j < 5; ++j) ix.x[j] = tr + 64 * j < ix.dcp ? dr[tr + 64 * j] : -1;
        const int32_t* od = p.order + (int64_t)(q0 + qi) * kDistinctRows;
#pragma unroll
        for (int j = 0; j < 2; ++j) ix.d[j] = od[tr + 64 * j];
    };
    auto load_dat = [&](const Idx& ix, Dat& v) {
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int s = tr + 64 * j;
            v.x[j] = u32x4w_t{0u, 0u, 0u, 0u};
            if ((uint32_t)ix.x[j] < N32)
                v.x[j] = *(const u32x4w_t*)(p.feats + ((int64_t)ix.x[j] * p.Ci + ci0) * 2 +
                                            16 * (tc ^ (2 * ((s >> 3) & 1))));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = tr + 64 * j;
            v.d[j] = u32x4w_t{0u, 0u, 0u, 0u};
            if (ix.d[j] >= 0)
                v.d[j] = *(const u32x4w_t*)(p.dout + ((int64_t)ix.d[j] * p.Co + co0) * 2 +
                                            16 * (tc ^ (2 * ((r >> 3) & 1))));
        }
        const uint8_t* sm = (const uint8_t*)(p.smap + (int64_t)(q0 + ix.qi) * K * kDistinctRows);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            v.s[j] = u32x4w_t{0u, 0u, 0u, 0u};
            if (16 * (t + kWtThreads * j) < K * kDistinctRows * 2)
                v.s[j] = *(const u32x4w_t*)(sm + 16 * (t + kWtThreads * j));
        }
    };
    auto store_dat = [&](const Idx& ix, const Dat& v, uint8_t* st) {
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int s = tr + 64 * j;
            if (s < ix.dcp) *(u32x4w_t*)(st + 64 * s + 16 * tc) = v.x[j];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) *(u32x4w_t*)(st + kWtDout + 64 * (tr + 64 * j) + 16 * tc) = v.d[j];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (16 * (t + kWtThreads * j) < K * kDistinctRows * 2)
                *(u32x4w_t*)(st + kWtCodes + 16 * (t + kWtThreads * j)) = v.s[j];
    };
    // transposing read: lane a of each 16-lane group addresses 4 channels
    // (4 (a & 3) ..) of row a >> 2 of four rows and receives channel a of the
    // four rows
    auto tr_read = [&](const uint8_t* rowp) -> bf16x4w_t {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4w_t*)rowp);
    };
    // one unit: B fragments of the four k-steps, then the wave's offsets
    auto compute = [&](int qi, int ps, const uint8_t* st) {
        const bool layered = (dcs[qi] & kLayerPasses) != 0u;
        const int q = q0 + qi;
        bf16x8w_t bfr[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const int r0 = 32 * s + 8 * g4 + (a >> 2);
                const int r1 = r0 + 4;
                const bf16x4w_t lo = tr_read(st + kWtDout + 64 * r0 + 32 * (cb ^ ((r0 >> 3) & 1)) + 8 * (a & 3));
                const bf16x4w_t hi = tr_read(st + kWtDout + 64 * r1 + 32 * (cb ^ ((r1 >> 3) & 1)) + 8 * (a & 3));
                bfr[s][cb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        // the half tile's block masks of every offset (lane k)
        const uint32_t mv = lane < K ? ((uint32_t)p.blkmask[(int64_t)(q >> 1) * K + lane] >> (8 * (q & 1))) & 0xFFu : 0u;
#pragma unroll
        for (int i = 0; i < kWtMaxOff; ++i) {
            const int k = wv + 4 * i;
            if (k >= K) break;
            if (layered && (k < 9 * ps || k >= 9 * ps + 9)) continue;
            const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)mv, k);
            if (!m) continue;
            // codes of rows 32 s + 8 g4 + 4 h + (a >> 2): element 2 s + (g4 >> 1)
            // of the 16 bytes at position 8 (8 (g4 & 1) + 4 h + (a >> 2))
            const uint8_t* cp = st + kWtCodes + k * (kDistinctRows * 2) + 16 * (8 * (g4 & 1) + (a >> 2));
            const u32x4w_t c0 = *(const u32x4w_t*)cp;
            const u32x4w_t c1 = *(const u32x4w_t*)(cp + 16 * 4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (!((m >> (2 * s)) & 3u)) continue;
                const uint32_t s0 = ((g4 >> 1) ? (c0[s] >> 16) : (c0[s] & 0xFFFFu)) >> 4;
                const uint32_t s1 = ((g4 >> 1) ? (c1[s] >> 16) : (c1[s] & 0xFFFFu)) >> 4;
                bf16x8w_t af[2];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const bf16x4w_t lo = tr_read(st + 64 * s0 + 32 * (hb ^ ((s0 >> 3) & 1)) + 8 * (a & 3));
                    const bf16x4w_t hi = tr_read(st + 64 * s1 + 32 * (hb ^ ((s1 >> 3) & 1)) + 8 * (a & 3));
                    af[hb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        acc[i][hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[hb], bfr[s][cb], acc[i][hb][cb], 0, 0, 0);
            }
        }
    };

    // the unit sequence: indices two units ahead, rows one
    Idx ia, ib;
    Dat dv;
    int cq = 0, cp = 0;     // the unit whose rows are in dv and indices in ia
    int q1 = 0, p1 = 0;     // the next one (indices in ib)
    int q2 = 0, p2 = 0;     // the one after
    if (nq > 0) {
        advance(q1, p1);
        q2 = q1;
        p2 = p1;
        if (q2 < nq) advance(q2, p2);
        load_idx(0, 0, ia);
        if (q1 < nq) load_idx(q1, p1, ib);
        load_dat(ia, dv);
    }
    int buf = 0;
    while (cq < nq) {
        uint8_t* st = stg + buf * kWtStage;
        store_dat(ia, dv, st);
        if (q1 < nq) load_dat(ib, dv);
        ia = ib;
        if (q2 < nq) load_idx(q2, p2, ib);
        const int pq = cq, pp = cp;
        cq = q1;
        cp = p1;
        q1 = q2;
        p1 = p2;
        if (q2 < nq) advance(q2, p2);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the stage is written
        barrier_only();
        compute(pq, pp, st);
        buf ^= 1;
    }

    // partials: lane (a, g4) holds rows 4 g4 .. + 3 (input channels), column a
    // (output channel) of each 16 x 16 block
#pragma unroll
    for (int i = 0; i < kWtMaxOff; ++i) {
        const int k = wv + 4 * i;
        if (k >= K) break;
        float* out = p.part + ((((int64_t)k * nti + ti) * nto + to) * p.nchunks + c) * (32 * 32);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) out[(16 * hb + 4 * g4 + e) * 32 + 16 * cb + a] = acc[i][hb][cb][e];
    }
}

// dw[k][ci][co] = sum over chunks of the partials, in chunk order; one RNE
// rounding to bf16 or plain fp32 store
template <bool BF16, int TI, int TO>
__global__ void __launch_bounds__(256) k_wgrad_reduce(const float* __restrict__ part, int K, int Ci, int Co,
                                                      int nchunks, void* dw) {
    const int64_t total = (int64_t)K * Ci * Co;
    const int nto = Co / TO;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int k = (int)(e / ((int64_t)Ci * Co));
        const int ci = (int)((e / Co) % Ci), co = (int)(e % Co);
        const float* src = part + (((int64_t)k * (Ci / TI) + ci / TI) * nto + co / TO) * nchunks * (TI * TO) +
                           (ci % TI) * TO + (co % TO);
        float s = 0.f;
        for (int c = 0; c < nchunks; ++c) s += src[(int64_t)c * (TI * TO)];
        if constexpr (BF16) {
            uint32_t u = __float_as_uint(s);
            uint16_t h;
            if ((u & 0x7fffffffu) > 0x7f800000u) {
                h = (uint16_t)((u >> 16) | 0x40u);
            } else {
                u += 0x7fffu + ((u >> 16) & 1u);
                h = (uint16_t)(u >> 16);
            }
            ((uint16_t*)dw)[e] = h;
        } else {
            ((float*)dw)[e] = s;
        }
    }
}

int tile_of(int C) { return C % 128 == 0 ? 128 : (C % 64 == 0 ? 64 : 32); }

// bf16 with a 128-channel input tile and a 64- or 128-channel output tile runs
// the grouped-offset kernel
bool wgrad_grouped(int dtype, int Ci, int Co) {
    return dtype == SPCONV_BF16 && tile_of(Ci) == 128 && tile_of(Co) >= 64;
}

template <bool BF16, int TI, int TO>
hipError_t launch_t(const WgradParams& p, void* dw, hipStream_t s) {
    if constexpr (BF16 && TI == 128 && TO >= 64) {
        if (p.nchunks > 0 && wgrad_grouped(SPCONV_BF16, p.Ci, p.Co)) {
            const int64_t nwg = (int64_t)p.nchunks * ((p.K + kWgGroup - 1) / kWgGroup) * (p.Ci / TI) * (p.Co / TO);
            k_wgrad_g<TI, TO><<<dim3((unsigned)nwg), dim3(kWgThreads), 0, s>>>(p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t total = (int64_t)p.K * p.Ci * p.Co;
            const int64_t blocks = (total + 255) / 256;
            k_wgrad_reduce<BF16, TI, TO><<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s>>>(
                p.part, p.K, p.Ci, p.Co, p.nchunks, dw);
            return hipGetLastError();
        }
    }
    if (p.nchunks > 0) {   // no chunks (no rows): the reduction writes zeros
        dim3 grid((unsigned)p.nchunks, (unsigned)p.K, (unsigned)((p.Ci / TI) * (p.Co / TO)));
        k_wgrad<BF16, TI, TO><<<grid, dim3(kWgThreads), 0, s>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t total = (int64_t)p.K * p.Ci * p.Co;
    const int64_t blocks = (total + 255) / 256;
    k_wgrad_reduce<BF16, TI, TO><<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s>>>(
        p.part, p.K, p.Ci, p.Co, p.nchunks, dw);
    return hipGetLastError();
}

template <bool BF16, int TI>
hipError_t launch_ti(const WgradParams& p, void* dw, hipStream_t s) {
    switch (tile_of(p.Co)) {
        case 128: return launch_t<BF16, TI, 128>(p, dw, s);
        case 64: return launch_t<BF16, TI, 64>(p, dw, s);
        default: return launch_t<BF16, TI, 32>(p, dw, s);
    }
}

template <bool BF16>
hipError_t launch_dt(const WgradParams& p, void* dw, hipStream_t s) {
    switch (tile_of(p.Ci)) {
        case 128: return launch_ti<BF16, 128>(p, dw, s);
        case 64: return launch_ti<BF16, 64>(p, dw, s);
        default: return launch_ti<BF16, 32>(p, dw, s);
    }
}

}  // namespace

bool wgrad_supported(int dtype, int Ci, int Co) {
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16) return false;
    return Ci >= 32 && Co >= 32 && Ci % 32 == 0 && Co % 32 == 0 && Ci <= 4096 && Co <= 4096;
}

// Row chunks: enough workgroups to fill the chip about four times over, and no
// more chunks than 128-row (64-row for fp32) units.
int wgrad_chunks(int64_t N, int K, int Ci, int Co, int dtype) {
    const int64_t Npad = round_up(N > 0 ? N : 1, kTileRows);
    const int64_t nunits = Npad / wg_rows(dtype == SPCONV_BF16);
    const int64_t tiles = (int64_t)K * (Ci / tile_of(Ci)) * (Co / tile_of(Co));
    int64_t nc = (1024 + tiles - 1) / tiles;
    if (wgrad_grouped(dtype, Ci, Co)) {
        // one workgroup per CU: about two rounds of 256, in a multiple of 8
        // chunks (one XCD's share each)
        const int64_t gtiles = (int64_t)((K + kWgGroup - 1) / kWgGroup) * (Ci / tile_of(Ci)) * (Co / tile_of(Co));
        nc = (512 + gtiles - 1) / gtiles;
        if (nc >= 8) nc = nc / 8 * 8;
    }
    if (nc > nunits) nc = nunits;
    return (int)(nc < 1 ? 1 : nc);
}

// Chunks of the distinct-row kernel: about two workgroups per CU over the
// (Ci / 32) x (Co / 32) channel slices, a multiple of 8 (one XCD's share
// each), at most kWtMaxHalves half tiles per chunk.
bool wgrad_tile_shape(int64_t N, int K, int Ci, int Co, int dtype) {
    return dtype == SPCONV_BF16 && N > 0 && K <= kDistinctMaxK && Ci % 32 == 0 && Co % 32 == 0;
}
int wgrad_tile_chunks(int64_t N, int Ci, int Co) {
    const int64_t nhalf = round_up(N > 0 ? N : 1, kTileRows) / kDistinctRows;
    const int64_t nsl = (int64_t)(Ci / 32) * (Co / 32);
    int64_t nc = (512 + nsl - 1) / nsl;
    if (nc >= 8) nc = nc / 8 * 8;
    const int64_t need = (nhalf + kWtMaxHalves - 1) / kWtMaxHalves;
    if (nc < need) nc = (need + 7) / 8 * 8;
    if (nc > nhalf) nc = nhalf;
    return (int)(nc < 1 ? 1 : nc);
}

size_t wgrad_workspace_bytes(int64_t N, int K, int Ci, int Co, int dtype) {
    int64_t nc = wgrad_chunks(N, K, Ci, Co, dtype);
    if (wgrad_tile_shape(N, K, Ci, Co, dtype)) nc = std::max<int64_t>(nc, wgrad_tile_chunks(N, Ci, Co));
    return (size_t)K * Ci * Co * 4 * (size_t)nc;
}

hipError_t launch_wgrad(const WgradArgs& a, hipStream_t stream) {
    if (!wgrad_supported(a.dtype, a.Ci, a.Co)) return hipErrorInvalidValue;
    // bf16 maps whose half tiles all have distinct-row lists: the list kernel,
    // except where the grouped kernel measured faster (128-channel multiples
    // on both sides: surf256 1.19 against 1.29 ms, though at 2.2x the HBM
    // traffic; at 128 -> 64, surf1024, the list kernel takes 8.3 ms against 10.3)
    if (wgrad_tile_shape(a.N, a.K, a.Ci, a.Co, a.dtype) && a.dcount && a.drow && a.smap && a.max_distinct >= 0 &&
        a.max_distinct <= kDistinctListCap && !(wgrad_grouped(a.dtype, a.Ci, a.Co) && a.Co % 128 == 0)) {
        WtParams q;
        q.feats = (const uint8_t*)a.feats;
        q.dout = (const uint8_t*)a.dout;
        q.order = a.order;
        q.blkmask = a.blkmask;
        q.dcount = a.dcount;
        q.drow = a.drow;
        q.smap = a.smap;
        q.part = (float*)a.workspace;
        q.N = a.N;
        q.K = a.K;
        q.Ci = a.Ci;
        q.Co = a.Co;
        q.nhalf = (int)(a.Npad / kDistinctRows);
        q.nchunks = wgrad_tile_chunks(a.N, a.Ci, a.Co);
        q.per_chunk = (q.nhalf + q.nchunks - 1) / q.nchunks;
        if (q.per_chunk > kWtMaxHalves) return hipErrorInvalidValue;
        const int64_t nwg = (int64_t)q.nchunks * (a.Ci / 32) * (a.Co / 32);
        k_wgrad_tile<<<dim3((unsigned)nwg), dim3(kWtThreads), 0, stream>>>(q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t total = (int64_t)a.K * a.Ci * a.Co;
        const int64_t blocks = (total + 255) / 256;
        k_wgrad_reduce<true, 32, 32><<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream>>>(
            q.part, a.K, a.Ci, a.Co, q.nchunks, a.dw);
        return hipGetLastError();
    }
    WgradParams p;
    p.feats = a.feats;
    p.dout = a.dout;
    p.nbr_m = a.nbr_m;
    p.order = a.order;
    p.blkmask = a.blkmask;
    p.part = (float*)a.workspace;
    p.N = a.N;
    p.Npad = a.Npad;
    p.K = a.K;
    p.Ci = a.Ci;
    p.Co = a.Co;
    p.nchunks = a.N > 0 ? wgrad_chunks(a.N, a.K, a.Ci, a.Co, a.dtype) : 0;
    const int64_t nunits = a.Npad / wg_rows(a.dtype == SPCONV_BF16);
    p.units_per_chunk = p.nchunks > 0 ? (int)((nunits + p.nchunks - 1) / p.nchunks) : 0;
    return a.dtype == SPCONV_BF16 ? launch_dt<true>(p, a.dw, stream) : launch_dt<false>(p, a.dw, stream);
}

}  // namespace spc
