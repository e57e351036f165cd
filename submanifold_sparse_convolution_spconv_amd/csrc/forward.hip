// Fused gather-GEMM-accumulate forward for gfx950.
//
//   out[n, co] = bias[co] + sum_k sum_ci feats[nbr[k, n], ci] * w[k, ci, co]
//
// (page "mlx_backend/sparse_conv_metal.py": module docstring formula, the kernel
// body's loop over k with the nbr >= N skip and fp32 accumulation, and the
// wrapper's layouts).  The page's kernel gives one thread per (n, co) and loops
// over scalars; here the same sum is computed as an output-stationary implicit
// GEMM on the matrix cores:
//
//  * A workgroup (4 waves) owns a tile of rows of the builder's schedule
//    (Morton order, rows mask-sorted in 256-row tiles) and BN output channels.
//    Each wave owns NB 16-row blocks and keeps their fp32 accumulators
//    (NB x BN/16 MFMA tiles) in registers across all K offsets.
//  * Per offset k, each wave gathers its rows' feature vectors straight from
//    feats into VGPRs in the MFMA operand layout (zero for the sentinel), while
//    the workgroup stages w[k][:, co0:co0+BN] into LDS (double-buffered, the
//    next offset's loads overlapping this offset's MFMAs).
//  * Offsets for which no row of the tile has a neighbour are skipped, and
//    within an offset each wave skips the MFMAs of 16-row blocks that are
//    entirely missing (the builder's per-(tile, k) block masks).
//  * bf16: v_mfma_f32_16x16x32_bf16, w staged transposed (ci contiguous) with
//    an XOR swizzle of 16-byte chunks so both the transposing writes and the
//    fragment reads spread over the LDS banks.
//    fp32: v_mfma_f32_16x16x4_f32, w staged in its natural layout.
//  * Epilogue: + bias in fp32, one round-to-nearest-even to the output type,
//    rows scattered back to caller order through the schedule.
//  * Mixed dtypes (the page's wrapper casts feats to w's dtype): the register
//    gather of each kernel also reads the other feature type.  The loaded words
//    stay raw in the look-ahead stages and are converted where the MFMAs take
//    them, so the cast adds no wait: fp32 -> bf16 rounds to nearest even, and
//    bf16 -> fp32 is exact.  Output follows w's dtype.  fp32 features into bf16
//    weights can instead be cast by a separate streaming pass into a caller
//    workspace, after which the bf16 kernels (LDS-staged at Ci = 128, 256) run
//    as usual: the page's order, and faster where the staged kernel applies.
// No atomics: every output element is written once by one lane, so results
// are deterministic.
#include "spconv_internal.h"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace spc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));

constexpr int kMaxK = 1024;

struct FwdParams {
    const void* feats;
    const int32_t* nbr_m;
    const int32_t* order;
    const uint16_t* blkmask;
    const uint32_t* dcount;  // distinct neighbour rows per tile (distinct-row kernel)
    const int32_t* drow;
    const uint16_t* smap;
    const void* w;
    const void* wpack;      // packed weights for the LDS-staged kernel, or NULL
    const float* bias;
    void* out;
    int64_t N, Npad;
    int K, Co, ntiles;
    int tpw;                // tiles per workgroup (LDS-staged bf16 kernel)
    uint32_t* queue;        // tile kernel: [next, done] counters per channel group, zero
};

// The LDS-staged bf16 kernel runs up to this many consecutive tiles per
// workgroup, with at most kMaxK offset-list entries over all of them.
constexpr int kMaxTPW = 4;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN
    const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// Raw registers of the feature values one lane gathers per load step, for
// feature element type FT (uint16_t = bf16 bits, or float), and their
// conversion to the MFMA operand of the kernel's own type.
//   bf16 kernel: 8 consecutive channels -> bf16x8 (fp32 rounded to nearest even)
//   fp32 kernel: 4 consecutive channels -> f32x4 (bf16 widened exactly)
template <typename FT> struct Gather8;
template <> struct Gather8<uint16_t> { typedef u32x4_t raw; };
template <> struct Gather8<float> { typedef u32x8_t raw; };
template <typename FT> struct Gather4;
template <> struct Gather4<float> { typedef f32x4_t raw; };
template <> struct Gather4<uint16_t> { typedef u32x2_t raw; };

// feats is only 16-byte aligned: eight floats come in as two 16-byte loads
__device__ __forceinline__ u32x4_t load8(const uint16_t* p) { return *(const u32x4_t*)p; }
__device__ __forceinline__ u32x8_t load8(const float* p) {
    const u32x4_t a = *(const u32x4_t*)p, b = *(const u32x4_t*)(p + 4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x8_t v) {
    u32x4_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(__uint_as_float(v[2 * e]), __uint_as_float(v[2 * e + 1]));
    return __builtin_bit_cast(bf16x8_t, r);
}
__device__ __forceinline__ f32x4_t as_f32x4(f32x4_t v) { return v; }
__device__ __forceinline__ f32x4_t as_f32x4(u32x2_t v) {
    return f32x4_t{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                   __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
}

// fp32 -> bf16 (round to nearest even), eight values per thread and step:
// two 16-byte loads, one 16-byte store.  n8 = element count / 8.
__global__ void __launch_bounds__(256) k_cast_bf16(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                   int64_t n8) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
        const u32x4_t a = src[2 * i], b = src[2 * i + 1];
        u32x4_t r;
        r[0] = pack_bf16x2(__uint_as_float(a[0]), __uint_as_float(a[1]));
        r[1] = pack_bf16x2(__uint_as_float(a[2]), __uint_as_float(a[3]));
        r[2] = pack_bf16x2(__uint_as_float(b[0]), __uint_as_float(b[1]));
        r[3] = pack_bf16x2(__uint_as_float(b[2]), __uint_as_float(b[3]));
        dst[i] = r;
    }
}

// Workgroup -> tile.  Consecutive workgroup ids are dealt round-robin to the
// 8 XCDs; give each XCD a contiguous run of tiles so that neighbouring tiles,
// which gather overlapping feature rows, share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
    const int x = bid & 7, i = bid >> 3;
    const int q = ntiles >> 3, r = ntiles & 7;
    return x * q + (x < r ? x : r) + i;
}

__device__ __forceinline__ int swz(int n) { return n ^ (n >> 3); }

// ---------------------------------------------------------------------------
// bf16 kernel.
//
// MFMA roles: srcA = w (M = 16 output channels), srcB = gathered feature rows
// (N = 16 rows of the schedule), K = 32 input channels per instruction.  The
// output tile D[m][n] then lands in lane l as D[4g+i][l%16] (g = l/16), i.e.
// four channels of one row.  The channels of the 16-wide srcA tile j are
// assigned as co(j, m) = (m/4)*4*NJ + 4j + m%4, so over the NJ tiles of a wave
// each lane holds 4*NJ *contiguous* channels of its row and the epilogue
// writes whole 16-byte pieces of out rows.
//
// w[k][:, co0:co0+BN] is staged in LDS in its natural (ci, co) layout with
// ds_write_b128; srcA fragments are read with the gfx950 transposing read
// ds_read_b64_tr_b16, which hands lane i of each 16-lane group element i%4 of
// the 8 bytes addressed by lane 4j+i/4 of the group (j = output element):
// lane a = 4*jj + q of group g addresses row ci = 32s + 8g + 4h + jj at
// channel co(j, 4q), and receives 4 consecutive ci of channel co(j, i).
// Rows are XOR-swizzled in 8-byte units so that those 16 row reads and the
// staging writes spread over the LDS banks.
//
// Template: CI input channels, BN channels per workgroup, NB 16-row blocks per
// wave, NWR x NWC waves (rows x channels), D = how many offsets ahead the
// feature gather runs (D+1 register stages), FT = feature element type.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

template <int BN>
__device__ __forceinline__ int unit_swz(int ci) {
    return ((ci & 3) | ((ci >> 1) & 4) | (ci & 16)) & (BN / 4 - 1);
}

template <int CI, int BN, int NB, int NWR, int NWC, int D, typename FT>
__global__ void __launch_bounds__(64 * NWR * NWC) k_fwd_bf16(FwdParams p) {
    typedef typename Gather8<FT>::raw Raw;
    constexpr int NT = 64 * NWR * NWC;
    constexpr int BM = NWR * NB * 16;
    constexpr int NS = CI / 32;                 // MFMA k-steps (32 ci each)
    constexpr int WCOLS = BN / NWC;             // channels per wave
    constexpr int NJ = WCOLS / 16;              // 16-channel MFMA tiles per wave
    constexpr int WCH = CI * BN / 8;            // 16-byte chunks of a staged w[k] slice
    constexpr int WPT = (WCH + NT - 1) / NT;
    constexpr int NST = D + 1;                  // feature register stages
    constexpr uint32_t TBITS = (1u << (NWR * NB)) - 1u;
    static_assert(NJ >= 2 && NJ % 2 == 0, "epilogue packs channel pairs");

    __shared__ __attribute__((aligned(16))) uint16_t ws[2][CI * BN];
    __shared__ uint16_t tmask[kMaxK];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wr = wave % NWR, wc = wave / NWR;
    const int g = lane >> 4;
    const int tile = xcd_tile(blockIdx.x, p.ntiles);
    const int64_t row0 = (int64_t)tile * BM;
    const int co0 = blockIdx.y * BN;
    // 16-row blocks are dealt to the waves round-robin: block b of wave wr is
    // block wr + b*NWR of the tile.  Rows are mask-sorted inside the tile, so
    // the blocks that are present for one offset form contiguous runs; the
    // interleave spreads each run over all waves (and SIMDs).
    auto brow = [&](int b) -> int64_t { return row0 + (int64_t)(wr + b * NWR) * 16; };
    const int wcol0 = wc * WCOLS;
    const int K = p.K;
    const uint32_t N32 = (uint32_t)p.N;
    const FT* __restrict__ feats = (const FT*)p.feats;
    const uint16_t* __restrict__ w = (const uint16_t*)p.w;
    const int Co = p.Co;

    {
        const int64_t mt = row0 / kTileRows;
        const int msh = (int)((row0 % kTileRows) / 16);
        for (int k = t; k < K; k += NT)
            tmask[k] = (uint16_t)((p.blkmask[mt * K + k] >> msh) & TBITS);
    }
    __syncthreads();

    // K <= 64: the offsets' block masks in lane k and the set of offsets
    // with any (wave-uniform), so that stepping to the next offset reads no LDS
    const bool kreg = K <= 64;
    const uint32_t tmv = lane < K ? tmask[lane] : 0u;
    const uint64_t tact = __ballot(tmv != 0u);
    auto next_k = [&](int k) {
        if (kreg) {
            const uint64_t rest = k + 1 >= 64 ? 0ull : tact & (~0ull << (k + 1));
            return rest ? (int)__builtin_ctzll(rest) : K;
        }
        for (++k; k < K; ++k)
            if (tmask[k]) return k;
        return K;
    };
    // every lane loads the neighbour of its row (lane & 15) of each block
    // itself (four lanes share each address) rather than taking it from the
    // loading lane with a cross-lane read: shell64 24.2 -> 23.2 us
    typedef int32_t NbIdx[NB];
    auto load_nbr = [&](int k, NbIdx& v) {
#pragma unroll
        for (int b = 0; b < NB; ++b) v[b] = p.nbr_m[(int64_t)k * p.Npad + brow(b) + (lane & 15)];
    };
    auto gather = [&](const NbIdx& nbv, Raw (&f)[NB][NS]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int32_t nb = nbv[b];
            const bool ok = (uint32_t)nb < N32;
            const FT* src = feats + (int64_t)(ok ? nb : 0) * CI + 8 * g;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                Raw v = load8(src + 32 * s);
                if (!ok) v = (Raw)0u;
                f[b][s] = v;
            }
        }
    };
    auto load_w = [&](int k, u32x4_t (&wreg)[WPT]) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = t + NT * i;
            if (WCH % NT == 0 || e < WCH) {
                const int ci = e / (BN / 8), c8 = e % (BN / 8);
                wreg[i] = *(const u32x4_t*)(w + ((int64_t)k * CI + ci) * Co + co0 + c8 * 8);
            }
        }
    };
    // staged row ci of BN channels, 8-byte units XOR-swizzled by unit_swz(ci)
    auto store_w = [&](const u32x4_t (&wreg)[WPT], uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = t + NT * i;
            if (WCH % NT == 0 || e < WCH) {
                const int ci = e / (BN / 8), c8 = e % (BN / 8);
                const int sw = unit_swz<BN>(ci);
                u32x4_t v = wreg[i];
                if (sw & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
                *(u32x4_t*)(dst + ci * BN + ((c8 ^ (sw >> 1)) << 3)) = v;
            }
        }
    };
    // srcA fragment: 8 consecutive ci (two transposing reads) of channel co(j, lane%16)
    const int a16 = lane & 15;
    const int jj = a16 >> 2, q = a16 & 3;
    auto read_wfrag = [&](const uint16_t* wsb, int s, int j) -> bf16x8_t {
        bf16x4_t lo, hi;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ci = 32 * s + 8 * g + 4 * h + jj;
            const int u = (wcol0 >> 2) + q * NJ + j;
            const uint16_t* ptr = wsb + ci * BN + ((u ^ unit_swz<BN>(ci)) << 2);
            bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(
                (__attribute__((address_space(3))) uint16_t*)ptr));
            if (h == 0) lo = v; else hi = v;
        }
        return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    f32x4_t acc[NB][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    Raw fr[NST][NB][NS];
    u32x4_t wreg[WPT];

    // queue of the next D+1 active offsets (K = none)
    int kq[NST];
    kq[0] = (kreg ? (tact & 1ull) != 0ull : tmask[0] != 0) ? 0 : next_k(0);
    if (kq[0] < K) {
#pragma unroll
        for (int i = 1; i < NST; ++i) kq[i] = kq[i - 1] < K ? next_k(kq[i - 1]) : K;
        const int kfill = kq[0];
        auto clampk = [&](int k) { return k < K ? k : kfill; };
        load_w(kq[0], wreg);
#pragma unroll
        for (int i = 0; i < D; ++i) {
            NbIdx v;
            load_nbr(clampk(kq[i]), v);
            gather(v, fr[i]);
        }
        NbIdx nbv_next;
        load_nbr(clampk(kq[D]), nbv_next);
        store_w(wreg, ws[0]);
        __syncthreads();
        int buf = 0;

        auto iter = [&](auto st_c) -> bool {
            constexpr int ST = decltype(st_c)::value;
            constexpr int SG = (ST + D) % NST;     // stage receiving the gather for kq[D]
            load_w(clampk(kq[1 < NST ? 1 : 0]), wreg);
            gather(nbv_next, fr[SG]);
            const int knew = kq[D] < K ? next_k(kq[D]) : K;
            load_nbr(clampk(knew), nbv_next);

            const uint32_t tm = kreg ? (uint32_t)__builtin_amdgcn_readlane((int)tmv, kq[0] < 64 ? kq[0] : 0) : tmask[kq[0]];
            uint32_t wb = 0;
#pragma unroll
            for (int b = 0; b < NB; ++b) wb |= ((tm >> (wr + b * NWR)) & 1u) << b;
            if (wb) {
                const uint16_t* wsb = ws[buf];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    bf16x8_t wf[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) wf[j] = read_wfrag(wsb, s, j);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (wb & (1u << b)) {
                            const bf16x8_t fv = as_bf16x8(fr[ST][b][s]);
#pragma unroll
                            for (int j = 0; j < NJ; ++j)
                                acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    wf[j], fv, acc[b][j], 0, 0, 0);
                        }
                    }
                }
            }
            const bool more = NST > 1 ? kq[1] < K : false;
            if (more) store_w(wreg, ws[buf ^ 1]);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < D; ++i) kq[i] = kq[i + 1];
            kq[D] = knew;
            buf ^= 1;
            return kq[0] < K;
        };
        for (;;) {
            if (!iter(std::integral_constant<int, 0>{})) break;
            if constexpr (NST > 1) {
                if (!iter(std::integral_constant<int, 1 % NST>{})) break;
            }
            if constexpr (NST > 2) {
                if (!iter(std::integral_constant<int, 2 % NST>{})) break;
            }
        }
    }

    // epilogue: + bias, one RNE rounding; lane holds channels
    // co0 + wcol0 + g*4*NJ + [0, 4*NJ) of row brow(b) + lane%16
    uint16_t* __restrict__ out = (uint16_t*)p.out;
    const int cbase = co0 + wcol0 + g * 4 * NJ;
    float bsv[4 * NJ];
#pragma unroll
    for (int c = 0; c < 4 * NJ; ++c) bsv[c] = p.bias ? p.bias[cbase + c] : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int64_t r = brow(b) + (lane & 15);
        const int32_t n_out = p.order[r];
        if (n_out >= 0) {
            uint16_t* dst = out + (int64_t)n_out * Co + cbase;
#pragma unroll
            for (int j = 0; j < NJ; j += 2) {
                u32x4_t v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jx = j + (e >> 1);
                    const int i0 = (e & 1) * 2;
                    const uint32_t lo = f32_to_bf16_rne(acc[b][jx][i0] + bsv[4 * jx + i0]);
                    const uint32_t hi = f32_to_bf16_rne(acc[b][jx][i0 + 1] + bsv[4 * jx + i0 + 1]);
                    v[e] = lo | (hi << 16);
                }
                *(u32x4_t*)(dst + 4 * j) = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 kernel with LDS-staged rows, for Ci = 128 and 256.
//
// The operand layout of v_mfma_f32_16x16x32_bf16 puts row r of a 16-row block
// in lanes r, r+16, r+32, r+48, so a load straight into operand registers has
// every group of four consecutive lanes touching four different rows; the
// vector memory address path then needs four times the cycles of a load in
// which each group of four lanes reads 64 contiguous bytes.  Here each wave
// copies its rows' feature vectors into a private LDS stage with 16-byte
// global->LDS DMA loads whose lane groups read 64 contiguous bytes of one row
// (64-byte segments), and reads operands back with
// ds_read_b128.  gfx950's LDS has 128 four-byte banks and serves a
// ds_read_b128 for 32 lanes per pass, so the 16-byte units (address / 16)
// mod 32 of each half-wave must all differ.  Instruction j of a block lands
// kDmaPitch = 1056 bytes (66 units, = 2 mod 32) after instruction j-1, and
// quad q of an instruction carries row 4((q >> 1) & 3) + (j & 3), segment
// (q & 1) + 2(q >> 3) + 4(j >> 2); the operand read of row n, group g then
// hits unit 2n + g + const, distinct over a half-wave.  Missing neighbours are
// written as zeros by the lanes themselves.
//
// The per-tile list of active offsets (offset and 16-row block mask) is
// compacted in LDS once, so the offset loop and the per-block skips are
// scalar branches.
// ---------------------------------------------------------------------------
constexpr int kDmaPitch = 1056;


// NWR = 8: one workgroup of 8 waves per CU, w double-buffered.  NWR = 4: two
// workgroups of 4 waves per CU (128-row tiles, w single-buffered, two
// barriers per offset), so that one workgroup's loads and barriers overlap
// the other's MFMAs.
// PK: w comes pre-packed (spconv_pack_weights) in exactly the staged plane
// layout, and each offset's slice is copied into LDS with 1 KB DMAs shared by
// all waves; otherwise the kernel transposes w itself (8 x 8 sub-tiles).
// Packed w slice (k, column tile) -> LDS planes of BN rows of 16 bytes (rows
// of odd planes XOR-swizzled, as in the packed copy).  The slice holds the BN
// rows of each input-channel group u back to back; they are copied in pieces
// of up to 1 KB (one 16-byte DMA per lane), piece pc to plane u = pc / PPP,
// row 64 (pc % PPP).
template <int CI, int BN>
struct WPieces {
    static constexpr int PPP = BN >= 64 ? BN / 64 : 1;     // pieces per plane
    static constexpr int LANES = BN >= 64 ? 64 : BN;      // lanes of one piece
    static constexpr int NP = (CI / 8) * PPP;             // pieces per slice
    static constexpr uint32_t SLICE = (uint32_t)CI * BN * 2;
};
template <int CI, int BN>
__device__ __forceinline__ void dma_w_piece(__amdgpu_buffer_rsrc_t rsrc, uint32_t slice_off, uint16_t* dst, int pc,
                                            int lane) {
    using P = WPieces<CI, BN>;
    const int u = pc / P::PPP, h = pc % P::PPP;
    if (P::LANES == 64 || lane < P::LANES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(dst + (u * BN + 64 * h) * 8), 16,
            slice_off + (uint32_t)(u * BN + 64 * h) * 16u + 16u * (uint32_t)lane, 0, 0, 0);
}

// Row of plane u that holds MFMA tile row r (= 16 j + m): rows of odd planes
// are XOR-swizzled by 16, so that the two lane groups of a half-wave, which
// read planes 4s + g of the same row index, fall on opposite halves of the
// 32 16-byte bank units.
__device__ __forceinline__ int wrow(int u, int r) { return r ^ (16 * (u & 1)); }

template <int CI, int BN, int NB, int NWR, bool PK>
__global__ void __launch_bounds__(64 * NWR, 8 / NWR) k_fwd_bf16_lds(FwdParams p) {
    constexpr int NT = 64 * NWR;
    constexpr int WB = NWR == 8 ? 2 : 1;         // staged w buffers
    constexpr int BM = NWR * NB * 16;
    constexpr int NS = CI / 32;                  // k-steps of 32 channels = DMA instructions per block
    constexpr int NJ = BN / 16;
    constexpr int STAGE_B = NS * kDmaPitch;      // bytes of one staged 16-row block
    constexpr int STAGE_W = NB * STAGE_B;        // bytes per wave
    constexpr int PLP = BN;                      // rows (16-byte units) per w plane
    constexpr int WPL = (CI / 8) * PLP * 8;      // uint16 elements of one staged w[k]
    constexpr int NSUB = (CI / 8) * (BN / 8);    // 8 x 8 staging sub-tiles per w[k]
    constexpr uint32_t TBITS = (1u << (NWR * NB)) - 1u;
    static_assert(CI % 128 == 0, "rows are staged in 4-row groups of 64-byte segments");
    static_assert(NJ >= 2 && NJ % 2 == 0, "epilogue packs channel pairs");
    static_assert(NSUB % 64 == 0 && NSUB <= NT, "whole waves stage w");
    static_assert(NB * NS <= 16, "row DMAs per wave");
    constexpr bool WALL = NSUB == NT;            // every wave takes part in the w staging

    __shared__ __attribute__((aligned(16))) uint16_t ws[WB][WPL];
    __shared__ __attribute__((aligned(16))) uint8_t stage[NWR * STAGE_W];
    __shared__ uint32_t klist[kMaxK];
    __shared__ int wcnt[NWR];
    __shared__ int32_t ord[kMaxTPW][BM];
    __shared__ float bsh[BN];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wr = __builtin_amdgcn_readfirstlane(t >> 6);
    const int g = lane >> 4;
    // this workgroup's tiles: tile0 .. tile0 + ntl - 1 (XCD-aware order)
    const int TPW = p.tpw;
    const int tile0 = xcd_tile(blockIdx.x, gridDim.x) * TPW;
    const int ntl = p.ntiles - tile0 < TPW ? p.ntiles - tile0 : TPW;
    const int co0 = blockIdx.y * BN;
    auto rowq = [&](int q) -> int64_t { return (int64_t)(tile0 + q) * BM; };
    auto brow = [&](int q, int b) -> int64_t { return rowq(q) + (int64_t)(wr + b * NWR) * 16; };
    const int K = p.K;
    const uint32_t N32 = (uint32_t)p.N;
    const uint16_t* __restrict__ w = (const uint16_t*)p.w;
    const int Co = p.Co;
    // feats as a buffer resource: N * CI * 2 < 2^32 bytes (checked by the
    // host); an offset of nbytes is out of range and DMAs zeros
    const uint32_t nbytes = N32 * (uint32_t)(2 * CI);
    const __amdgpu_buffer_rsrc_t frsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.feats), (short)0, (int)nbytes, 0x00020000);

    // bias and the row order of the workgroup's tiles, for the epilogues
    for (int i = t; i < BN; i += NT) bsh[i] = p.bias ? p.bias[co0 + i] : 0.f;
    for (int i = t; i < ntl * BM; i += NT) ord[i / BM][i % BM] = p.order[(int64_t)tile0 * BM + i];

    // compact the tiles' active offsets, tile by tile in offset order:
    // klist[i] = k | q << 10 | mask << 16 for tile q.  Offset 0 is kept even
    // with no active block, so that every tile has an entry (and an epilogue).
    int kcount = 0;
    for (int base = 0; base < ntl * K; base += NT) {
        const int e = base + t;
        const int q = e / K, k = e - q * K;
        uint32_t m = 0;
        bool keep = false;
        if (e < ntl * K) {
            const int64_t r0 = rowq(q);
            m = (uint32_t)(p.blkmask[(r0 / kTileRows) * K + k] >> (int)((r0 % kTileRows) / 16)) & TBITS;
            keep = m != 0u || k == 0;
        }
        const uint64_t bal = __ballot(keep);
        const int rank = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wcnt[wr] = __popcll(bal);
        __syncthreads();
        int off = kcount, tot = kcount;
#pragma unroll
        for (int v = 0; v < NWR; ++v) {
            off += v < wr ? wcnt[v] : 0;
            tot += wcnt[v];
        }
        if (keep) klist[off + rank] = (uint32_t)k | ((uint32_t)q << 10) | (m << 16);
        kcount = tot;
        __syncthreads();
    }

    uint8_t* const wstage = stage + wr * STAGE_W;
    // lane l needs the neighbours of rows 4 * ((l >> 3) & 3) + 0..3 of each
    // block.  With two blocks one 16-byte load serves both: lanes 0-31 read
    // block 0's rows, lanes 32-63 block 1's, and v_permlane32_swap hands each
    // half the other's values when they are used (expand_nq), not when they
    // arrive.
    const int a4 = 4 * ((lane >> 3) & 3);
    auto load_nq = [&](uint32_t e, u32x4_t& raw) {   // entry e: offset e & 1023 of tile (e >> 10) & 63
        raw = *(const u32x4_t*)(p.nbr_m + (int64_t)(e & 1023u) * p.Npad + brow((int)((e >> 10) & 63u), NB == 2 ? (lane >> 5) : 0) + a4);
    };
    auto expand_nq = [&](const u32x4_t& raw, u32x4_t (&nq)[NB]) {
        if constexpr (NB == 2) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const auto sw = __builtin_amdgcn_permlane32_swap(raw[d], raw[d], false, false);
                nq[0][d] = sw[0];   // lanes 0-31's values (block 0) in every lane
                nq[1][d] = sw[1];   // lanes 32-63's values (block 1) in every lane
            }
        } else {
            nq[0] = raw;
        }
    };
    // byte offset in the row of lane l's 16 bytes: segment ((l >> 2) & 1) + 2(l >> 5)
    const uint32_t seg_off = 64u * (uint32_t)(((lane >> 2) & 1) + 2 * (lane >> 5)) + 16u * (uint32_t)(lane & 3);
    // row DMAs of the blocks in mask m; missing neighbours get zeros (out of
    // range offset), blocks outside m are not loaded (their MFMAs are skipped)
    auto stage_rows = [&](uint32_t m, const u32x4_t (&nq)[NB]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!((m >> (wr + b * NWR)) & 1u)) continue;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint32_t nb = nq[b][j & 3];
                const uint32_t off = nb < N32 ? nb * (uint32_t)(2 * CI) + seg_off + 256u * (uint32_t)(j >> 2) : nbytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    frsrc, (__attribute__((address_space(3))) void*)(wstage + b * STAGE_B + j * kDmaPitch), 16, off,
                    0, 0, 0);
            }
        }
    };
    // operand of k-step s for lane (n, g): row n, channels 32s + 8g .. +7
    const int n16 = lane & 15;
    const int rd_base = (n16 & 3) * kDmaPitch + 128 * (n16 >> 2) + 16 * g;
    // blocks outside the offset's mask m were not staged and are not read
    auto read_rows = [&](bf16x8_t (&f)[NB][NS], uint32_t m) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!((m >> (wr + b * NWR)) & 1u)) continue;
            const uint8_t* sb = wstage + b * STAGE_B + rd_base;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                f[b][s] = *(const bf16x8_t*)(sb + (s >> 2) * 4 * kDmaPitch + 64 * (s & 1) + 512 * ((s >> 1) & 1));
        }
    };
    // w[k][:, co0:co0+BN] is staged transposed: plane u (channels 8u..8u+7)
    // holds one 16-byte unit per output channel, at row wrow(u, 16j + m) for
    // channel co(j, m) = (m >> 2) 4NJ + 4j + (m & 3), so that the A operand of
    // tile j, k-step s is one ds_read_b128 at plane 4s + g, row
    // wrow(4s + g, 16j + m): the two lane groups of a half-wave fall on
    // opposite halves of the banks.
    // Staging: thread t < NSUB loads an 8 x 8 sub-tile (8 input channels of
    // 8 consecutive output channels) and transposes it in registers.
    const int scb = t / (BN / 8), sq8 = t % (BN / 8);
    const bool stager = WALL || t < NSUB;
    auto load_w1 = [&](int k, int r, u32x4_t (&wreg)[8]) {
        wreg[r] = *(const u32x4_t*)(w + ((int64_t)k * CI + 8 * scb + r) * Co + co0 + 8 * sq8);
    };
    auto store_w = [&](const u32x4_t (&wreg)[8], uint16_t* dst) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int co = 8 * sq8 + c;
            const int row = 16 * ((co >> 2) & (NJ - 1)) + 4 * (co / (4 * NJ)) + (co & 3);
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_perm(wreg[2 * e + 1][c >> 1], wreg[2 * e][c >> 1], sel);
            *(u32x4_t*)(dst + (scb * PLP + wrow(scb, row)) * 8) = v;
        }
    };
    // packed w: slice (k, co tile) at byte (k * ntiles_co + tile) * CI * BN * 2
    using WP = WPieces<CI, BN>;
    const uint32_t nct = gridDim.y;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(PK ? p.wpack : p.w), (short)0, (int)(PK ? (uint32_t)p.K * nct * WP::SLICE : 0u),
        0x00020000);
    auto dma_w = [&](int k, uint16_t* dst) {
        const uint32_t slice_off = ((uint32_t)k * nct + blockIdx.y) * WP::SLICE;
#pragma unroll
        for (int c = wr; c < WP::NP; c += NWR) dma_w_piece<CI, BN>(wrsrc, slice_off, dst, c, lane);
    };
    // plane 4s + g has the parity of g: row 16j + n16 of it is stored at
    // 16 (j ^ (g & 1)) + n16
    const int wf_e = (g * PLP + n16 + 16 * (g & 1)) * 8;          // even tiles j
    const int wf_o = (g * PLP + n16 + 16 * ((g & 1) ^ 1)) * 8;    // odd tiles j
    auto read_wfrag = [&](const uint16_t* wsb, int s, int j) -> bf16x8_t {
        return *(const bf16x8_t*)(wsb + ((j & 1) ? wf_o : wf_e) + (4 * s * PLP + 16 * (j & ~1)) * 8);
    };

    f32x4_t acc[NB][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // epilogue of tile q: + bias, one RNE rounding, store through the row
    // order; lane holds channels co0 + g*4*NJ + [0, 4*NJ) of row
    // brow(q, b) + lane%16.  The accumulators are cleared for the next tile.
    uint16_t* __restrict__ out = (uint16_t*)p.out;
    const int cl = g * 4 * NJ;          // first channel of this lane, within the tile
    auto epilogue = [&](int q) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int32_t n_out = ord[q][(wr + b * NWR) * 16 + (lane & 15)];
            if (n_out >= 0) {
                uint16_t* dst = out + (int64_t)n_out * Co + co0 + cl;
#pragma unroll
                for (int j = 0; j < NJ; j += 2) {
                    u32x4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jx = j + (e >> 1);
                        const int i0 = (e & 1) * 2;
                        v[e] = pack_bf16x2(acc[b][jx][i0] + bsh[cl + 4 * jx + i0],
                                           acc[b][jx][i0 + 1] + bsh[cl + 4 * jx + i0 + 1]);
                    }
                    *(u32x4_t*)(dst + 4 * j) = v;
                }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };

    if (kcount > 0) {
        auto entry = [&](int i) -> uint32_t {
            return i < kcount ? (uint32_t)__builtin_amdgcn_readfirstlane((int)klist[i]) : 0u;
        };
        uint32_t e_cur = entry(0), e_nxt = entry(1);
        u32x4_t nraw, nq[NB];
        u32x4_t wreg[8];
        auto load_w = [&](int k) {
            if (PK) return;
            if (stager) {
#pragma unroll
                for (int r = 0; r < 8; ++r) load_w1(k, r, wreg);
            }
        };
        bf16x8_t fr[NB][NS];
        load_nq(e_cur, nraw);
        load_w((int)(e_cur & 1023u));
        if constexpr (PK) dma_w((int)(e_cur & 1023u), ws[0]);
        expand_nq(nraw, nq);
        stage_rows(e_cur >> 16, nq);
        load_nq(e_nxt, nraw);    // e_nxt = 0 when absent: offset 0 of tile 0, no blocks
        if constexpr (!PK) {
            if (stager) store_w(wreg, ws[0]);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wave's DMAs have landed
        read_rows(fr, e_cur >> 16);
        __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0)
        __syncthreads();
        int buf = 0;
        int q_acc = 0;   // tile whose outputs the accumulators hold
        for (int i = 0; i < kcount; ++i) {
            const uint32_t m = e_cur >> 16;
            const bool more = i + 1 < kcount;
            const uint32_t e_nn = entry(i + 2);
            const int q_cur = (int)((e_cur >> 10) & 63u);
            // The next offset's loads go out first (row DMAs, w, the neighbour
            // indices of the offset after), then this offset's MFMAs.  Its
            // rows were read into fr before the previous barrier.
            if (more) {
                expand_nq(nraw, nq);
                stage_rows(e_nxt >> 16, nq);
                load_w((int)(e_nxt & 1023u));
                if constexpr (PK && WB == 2) dma_w((int)(e_nxt & 1023u), ws[buf ^ 1]);
            }
            load_nq(e_nn, nraw);
            // first offset of the next tile: finish the previous one while
            // this offset's loads are in flight
            if (q_cur != q_acc) {
                epilogue(q_acc);
                q_acc = q_cur;
            }
            const uint16_t* wsb = ws[buf];
            // a wave with no active block at this offset reads no w fragments
            // (scalar branch: m and wr are wave-uniform)
            uint32_t wact = 0;
#pragma unroll
            for (int b = 0; b < NB; ++b) wact |= (m >> (wr + b * NWR)) & 1u;
            if (wact) {
                // w fragments are read one k-step ahead of the MFMAs that use them
                bf16x8_t wf[2][NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) wf[0][j] = read_wfrag(wsb, 0, j);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s + 1 < NS) {
#pragma unroll
                        for (int j = 0; j < NJ; ++j) wf[(s + 1) & 1][j] = read_wfrag(wsb, s + 1, j);
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if ((m >> (wr + b * NWR)) & 1u) {
#pragma unroll
                            for (int j = 0; j < NJ; ++j)
                                acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s & 1][j], fr[b][s],
                                                                                    acc[b][j], 0, 0, 0);
                        }
                    }
                }
            }
            if constexpr (WB == 2) {
                if constexpr (!PK) {
                    if (more && stager) store_w(wreg, ws[buf ^ 1]);
                }
                // the next offset's rows (and, packed, its w) have landed:
                // read the rows now, while other waves finish their MFMAs
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                if (more) read_rows(fr, e_nxt >> 16);
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): stage free for the next DMAs
                __syncthreads();
                buf ^= 1;
            } else {
                __syncthreads();                      // every wave is done with w of this offset
                if constexpr (PK) {
                    if (more) dma_w((int)(e_nxt & 1023u), ws[0]);
                } else {
                    if (more && stager) store_w(wreg, ws[0]);
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);
                if (more) read_rows(fr, e_nxt >> 16);
                __builtin_amdgcn_s_waitcnt(0xC07F);
                __syncthreads();
            }
            e_cur = e_nxt;
            e_nxt = e_nn;
        }
        epilogue(q_acc);
    }
}


// ---------------------------------------------------------------------------
// bf16 tile kernel (Ci = 128): each tile's distinct neighbour rows staged once.
//
// A tile here is a half tile of the schedule (128 rows, sorted by validity
// mask among themselves).  The builder lists, per tile, the distinct rows
// that its rows have as present neighbours (about 1.9 per row on the surface
// workloads) and, per (offset, row), the code of its neighbour's slot among
// them.  A workgroup copies a tile's distinct rows (all 128 channels) into LDS
// once, then runs every active offset of the tile against them; the MFMA
// operands of a (block, offset) are read from LDS through the slot codes.
// L2 -> LDS traffic per tile is one copy of each distinct row instead of one
// per (offset, row).  LDS holds kDistinctCap rows; the rare tile with more
// is staged in three passes, one per layer of nine offsets, each with its
// own rows.
//
// Two persistent workgroups per CU, each of four waves (one per SIMD) and
// 80 KB of LDS, so that one workgroup's staging and epilogue overlap the
// other's MFMA work.  Every wave owns all 8 blocks of the tile and 64 output
// channels, with the fp32 accumulators (8 blocks x 4 MFMA tiles) in registers.
// BN = 128: wave (kw, cw) = (w >> 1, w & 1) takes k-steps 2kw, 2kw + 1 of
// channel group cw; BN = 64: wave w takes k-step w.  The waves holding
// partial sums of the same outputs add them through LDS when the tile ends.
// There is no barrier inside the offset loop: each wave reads its w fragments
// and slot codes for the next active offset straight from L2 into registers
// (w packed so that every fragment is one contiguous 1 KB wave load), and its
// row fragments one block ahead, across offset boundaries.
//
// Staged rows: slot s at s * 256 bytes; its 16-byte chunk c (channels 8c ..
// 8c + 7) is stored at chunk c ^ f(s), f(s) = 2 ((s >> 1) & 7), so that the
// 32 lanes of a half-wave (16 rows, two chunks each) hit distinct banks for
// rows with consecutive slots; slot code v = (s << 4) | f(s) gives the byte
// address of chunk c as (v ^ c) << 4.  Slot kDistinctCap is a row of zeros
// (missing neighbours).
//
// Tiles without lists (a layer over the cap; maps of more than
// kDistinctMaxK offsets; maps whose lists are not known) take the DIRECT
// instantiation: the rows of two active offsets at a time are
// staged as they are (slot 128 c + row) with slot codes made in the kernel,
// between barriers, and the same per-offset code runs.
//
// Every output sums its terms in the same order whatever the tile or mode:
// offsets ascending, within an offset the wave's k-steps ascending (inside
// the MFMA in its fixed order), then the partial sums of the k-step groups
// ((0 + 1) for BN = 128; ((0 + 1) + (2 + 3)) for BN = 64), then the bias,
// and one rounding to bf16.
// ---------------------------------------------------------------------------
template <int BN>
struct TileCfg {
    static constexpr int NW = 4;                       // waves, one per SIMD
    static constexpr int WGS = 2;                      // workgroups per CU
    static constexpr int R = kDistinctRows;            // rows per tile
    static constexpr int KS = BN / 64;                 // k-steps per wave and offset
    static constexpr int NKW = 4 / KS;                 // waves over the four k-steps
    static constexpr int NCW = BN / 64;                // 64-channel groups per workgroup
    static constexpr int NRH = 1;                      // row groups
    static constexpr int NBW = R / 16;                 // 16-row blocks per wave
    static constexpr int NSV = NBW / 8;                // 16-byte slot-code loads per offset
    static constexpr int CAP = kDistinctCap;           // staged rows; slot CAP is the zero row
    static constexpr int ROWB = (CAP + 1) * 256;       // row stage bytes
    static constexpr int RED = NW * (NBW / 2) * 4 * 1024;   // partial-sum exchange of one round
    static constexpr int DSM = 2 * R * 256;            // DIRECT: slot codes of the staged pair
    static constexpr int RD = 1;                       // row fragments read this many blocks ahead
    static constexpr int NFR = 2;                      // row fragment buffers (divides NBW, > RD)
    static constexpr int NX = (CAP / 4 / NW + 15) / 16;   // row-index registers per lane for the staging
    static_assert(BN == 64 || BN == 128, "64 output channels per wave");
    static_assert(NKW * NCW == NW && NBW == 8 && R % (4 * NW) == 0, "wave layout");
    static_assert(RED <= CAP * 256 && DSM + 2 * R * 2 <= CAP * 256, "exchange and direct stage below the zero row");
    static_assert(ROWB + 4 * BN + 256 + 16 <= 160 * 1024 / WGS, "LDS");
};

template <int BN, bool DIRECT>
__global__ void __launch_bounds__(64 * TileCfg<BN>::NW, TileCfg<BN>::WGS) k_fwd_bf16_tile(FwdParams p) {
    using C = TileCfg<BN>;
    constexpr int KS = C::KS, NCW = C::NCW, CAP = C::CAP, NW = C::NW, NBW = C::NBW, NKW = C::NKW, R = C::R;
    constexpr int LCAP = kDistinctListCap;
    constexpr int NT = 64 * NW;
    typedef std::integral_constant<int, 0> P0;
    typedef std::integral_constant<int, 1> P1;

    __shared__ __attribute__((aligned(1024))) uint8_t rows[C::ROWB];
    __shared__ __attribute__((aligned(16))) float bsh[BN];
    __shared__ uint32_t next_s;           // the tile after the current one
    __shared__ __attribute__((aligned(256))) uint32_t dump[64];   // DMA target nobody reads
    uint8_t* const sml = rows + C::DSM;   // DIRECT: slot codes of the staged pair

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int g = lane >> 4, n16 = lane & 15;
    // wave wv = kw NCW + cw: k-steps from KS kw, channel group cw
    const int cw = wv % NCW, kw = wv / NCW;
    constexpr int rh = 0;
    const uint32_t cc = (uint32_t)(4 * KS * kw + g);   // chunk of this lane's first k-step
    const int K = p.K;
    const int Co = p.Co;
    const int NCG = Co / 64;
    const int cg = (int)blockIdx.y * NCW + cw;         // this wave's 64-channel group
    const uint32_t N32 = (uint32_t)p.N;
    const uint8_t* __restrict__ feats = (const uint8_t*)p.feats;
    const uint8_t* __restrict__ wpk = (const uint8_t*)p.wpack;

    for (int i = t; i < BN; i += NT) bsh[i] = p.bias ? p.bias[(int)blockIdx.y * BN + i] : 0.f;
    if (t < 16) *(u32x4_t*)(rows + CAP * 256 + 16 * t) = u32x4_t{0u, 0u, 0u, 0u};

    // tiles of this workgroup: the XCD's contiguous run of tiles, dealt
    // round-robin to its workgroups
    const int G = (int)gridDim.x, xcd = (int)(blockIdx.x & 7u), wi = (int)(blockIdx.x >> 3);
    const int Wx = G / 8 + (xcd < G % 8 ? 1 : 0);
    const int64_t before = (int64_t)xcd * (G / 8) + (xcd < G % 8 ? xcd : G % 8);
    const int run0 = (int)((int64_t)p.ntiles * before / G);
    const int run1 = (int)((int64_t)p.ntiles * (before + Wx) / G);

    // --- operands -----------------------------------------------------------
    typedef bf16x8_t WFrag[KS][4];
    typedef bf16x8_t RFrag[KS];
    WFrag wb[2];
    u32x4_t svb[2][C::NSV];
    constexpr int RD = C::RD, NFR = C::NFR;
    static_assert(NBW % NFR == 0 && NFR > RD, "row fragment buffers");
    RFrag fr[NFR];
    f32x4_t acc[NBW][4];

    // w fragments of offset k: fragment (k, cg, k-step, j) is 1 KB at
    // (((k NCG + cg) 4 + k-step) 4 + j) KB, lane l's 16 bytes at 16 l
    auto load_w = [&](int k, WFrag& w) __attribute__((always_inline)) {
        const uint8_t* src = wpk + ((((size_t)k * NCG + cg) * 4 + KS * kw) * 4) * 1024 + 16 * lane;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[ks][j] = *(const bf16x8_t*)(src + (ks * 4 + j) * 1024);
    };
    // slot codes of this lane's row n16 in the tile's blocks ([n16][b], 16
    // bytes): from the map's slot lists (offset smo of tile sv_tile), or, in
    // DIRECT mode, from the staged pair's codes in LDS (position smo)
    int64_t sv_tile = 0;
    auto load_sv = [&](int smo, u32x4_t (&sv)[C::NSV]) __attribute__((always_inline)) {
        const uint8_t* src;
        if constexpr (DIRECT)
            src = sml + smo * (2 * R) + n16 * 16;
        else
            src = (const uint8_t*)p.smap + ((size_t)sv_tile * K + smo) * (2 * R) + n16 * 16;
#pragma unroll
        for (int x = 0; x < C::NSV; ++x) sv[x] = *(const u32x4_t*)(src + 16 * x);
    };
    auto read_rows = [&](const u32x4_t (&sv)[C::NSV], int b, RFrag& f) __attribute__((always_inline)) {
        const uint32_t word = sv[b >> 3][(b >> 1) & 3];
        const uint32_t code = (b & 1) ? (word >> 16) : (word & 0xFFFFu);
        const uint32_t a0 = (code ^ cc) << 4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) f[ks] = *(const bf16x8_t*)(rows + (a0 ^ (64u * ks)));
    };
    auto mfma_block = [&](int b, const RFrag& f, const WFrag& w) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[ks][j], f[ks], acc[b][j], 0, 0, 0);
    };
    // One active offset (mask m, slot codes at sml position smo, w in wb[P]).
    // If there is a next one (mask mn, position smon), its w and slot codes
    // are requested first and its first RD blocks' rows read during this
    // offset's last RD blocks.  Row fragments of block b live in fr[b % NFR].
    // The loads and reads are issued whether or not the block is active (an
    // inactive block's slot codes all name the zero row), so that their
    // counts, and with them the waits the compiler places, are fixed.
    auto step = [&](auto PC, uint32_t m, int kn, int smon) __attribute__((always_inline)) {
        constexpr int P = decltype(PC)::value;
        load_sv(smon, svb[P ^ 1]);
        load_w(kn, wb[P ^ 1]);
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            const int nb = b + RD;
            if (nb < NBW)
                read_rows(svb[P], nb, fr[nb % NFR]);
            else
                read_rows(svb[P ^ 1], nb - NBW, fr[nb % NFR]);
            if ((m >> b) & 1u) mfma_block(b, fr[b % NFR], wb[P]);
        }
    };
    // first offset of a run: its w and slot codes (unless already
    // requested), and its first RD blocks
    auto start = [&](int k, int smo, bool requested) __attribute__((always_inline)) {
        if (!requested) {
            load_sv(smo, svb[0]);
            load_w(k, wb[0]);
        }
#pragma unroll
        for (int b = 0; b < RD; ++b) read_rows(svb[0], b, fr[b]);
    };
    // the wave's bits of a tile block mask: every block
    auto wave_bits = [&](uint32_t m) -> uint32_t { return m; };
    // block mask of tile q at offset kb + lane (its half of the 16-bit mask
    // of the schedule's 256-row tile)
    auto tile_mask = [&](int64_t q, int kb) -> uint32_t {
        static_assert(kTileRows == 2 * R, "two tiles per mask");
        // (a 32-bit index: no 64-bit lane address kept across the tile loop)
        return (lane < 32 && kb + lane < K)
                   ? ((uint32_t)p.blkmask[(uint32_t)((q >> 1) * K + kb) + (uint32_t)lane] >> (8 * (int)(q & 1))) & 0xFFu
                   : 0u;
    };
    // runs over the active offsets listed in the bit set `act` (bit i: offset
    // kb + i, mask in lane i of mv), slot positions given by smpos(i).  After
    // the last one the loads of a next offset go to the last one again.
    auto run = [&](uint64_t act, int kb, uint32_t mv, auto smpos, bool requested) __attribute__((always_inline)) {
        int i0 = __builtin_ctzll(act);
        act &= act - 1;
        uint32_t m0 = wave_bits((uint32_t)__builtin_amdgcn_readlane((int)mv, i0));
        start(kb + i0, smpos(i0), requested);
        for (;;) {
            const bool h1 = act != 0;
            const int i1 = h1 ? __builtin_ctzll(act) : i0;
            act &= act - 1;
            const uint32_t m1 = wave_bits((uint32_t)__builtin_amdgcn_readlane((int)mv, i1));
            step(P0{}, m0, kb + i1, smpos(i1));
            if (!h1) break;
            const bool h2 = act != 0;
            const int i2 = h2 ? __builtin_ctzll(act) : i1;
            act &= act - 1;
            const uint32_t m2 = wave_bits((uint32_t)__builtin_amdgcn_readlane((int)mv, i2));
            step(P1{}, m1, kb + i2, smpos(i2));
            if (!h2) break;
            m0 = m2;
            i0 = i2;
        }
    };

    // --- epilogue -----------------------------------------------------------
    uint16_t* __restrict__ out = (uint16_t*)p.out;
    f32x4_t* red = (f32x4_t*)rows;
    int32_t ordv[2 * (NBW / 2 / C::NKW)];
    // Epilogue, in two rounds of NBW / 2 blocks: every wave copies its
    // partial sums of the round's blocks into its exchange area (wave wv's,
    // NBW / 2 blocks x 4 MFMA tiles), then each wave finishes its share of the
    // round's blocks of its (row group, channel group) from the areas alone.
    // The accumulators are read once each, at fixed places, so they stay in
    // AGPRs; which blocks a wave finishes only changes LDS addresses.
    constexpr int HB = NBW / 2;             // blocks per round
    constexpr int HF = HB / NKW;            // of them finished by each wave
    auto put_round = [&](auto R) __attribute__((always_inline)) {
        constexpr int r = decltype(R)::value;
#pragma unroll
        for (int bi = 0; bi < HB; ++bi) {
#pragma unroll
            for (int j = 0; j < 4; ++j) red[((wv * HB + bi) * 4 + j) * 64 + lane] = acc[HB * r + bi][j];
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto sync_lds = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        barrier_only();
    };
    // blocks HB r + fb .. + HF - 1 of the wave's row and channel groups: the
    // NKW partial sums (wave (rh, u, cw)'s in area (rh NKW + u) NCW + cw)
    // added in the fixed order, bias, one rounding; 32 bytes per lane
    // (channels 16 g .. 16 g + 15 of the group) of rows 16 b + n16, through
    // the row order
    const int fb = HF * kw;   // this wave's first block of a round
    auto finish_round = [&](int r) __attribute__((always_inline)) {
        uint16_t* obase = out + (int)blockIdx.y * BN + cw * 64 + 16 * g;
#pragma unroll
        for (int bi = 0; bi < HF; ++bi) {
            u32x4_t v[2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4_t pt[NKW];
#pragma unroll
                for (int u = 0; u < NKW; ++u)
                    pt[u] = red[((((rh * NKW + u) * NCW + cw) * HB + fb + bi) * 4 + j) * 64 + lane];
                f32x4_t sum;
                if constexpr (NKW == 2) sum = pt[0] + pt[1];
                else sum = (pt[0] + pt[1]) + (pt[2] + pt[3]);
                const f32x4_t s = sum + *(const f32x4_t*)&bsh[cw * 64 + 16 * g + 4 * j];
                v[j >> 1][2 * (j & 1)] = pack_bf16x2(s[0], s[1]);
                v[j >> 1][2 * (j & 1) + 1] = pack_bf16x2(s[2], s[3]);
            }
            const int32_t n = ordv[r * HF + bi];
            if (n >= 0) {
                uint16_t* dst = obase + (int64_t)n * Co;
                *(u32x4_t*)dst = v[0];
                *(u32x4_t*)(dst + 8) = v[1];
            }
        }
    };
    // output rows of the blocks this wave finishes: tile block NRH (HB r + fb
    // + i) + rh
    auto load_order = [&](int64_t tq) __attribute__((always_inline)) {
        // (32-bit indices, Npad < 2^31, and the lane's part recomputed here:
        // no lane offset kept across the tile loop)
        uint32_t lid;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
        const uint32_t o = (uint32_t)(tq * R) + (uint32_t)(16 * (C::NRH * fb + rh)) + (lid & 15u);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < HF; ++i) ordv[r * HF + i] = p.order[o + (uint32_t)(16 * C::NRH * (HB * r + i))];
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, 1> I1;
    auto epilogue = [&]() __attribute__((always_inline)) {
        sync_lds();   // every wave is past its last row read
        put_round(I0{});
        sync_lds();
        finish_round(0);
        sync_lds();
        put_round(I1{});
        sync_lds();
        finish_round(1);
        sync_lds();   // the exchange area is read: the next tile may stage
    };

    // --- tiles --------------------------------------------------------------
    // Tiles come from a queue (one counter per channel group): every
    // workgroup starts with tile blockIdx.x and takes the next one, gx + the
    // counter's old value, while staging the current one, so that the
    // workgroups stay busy until the queue is empty whatever each tile costs.
    // The last workgroup of a channel group to finish sets its counters back
    // to zero for the next launch that uses them.  The DIRECT instantiation
    // (few tiles) deals its tiles statically instead: the XCD's contiguous
    // run, round-robin to its workgroups.
    uint32_t* const qctr = p.queue + 2 * blockIdx.y;
    const bool lead = wv == 0 && lane == 0;
    __syncthreads();
    // block masks and distinct-row indices of the next tile, requested one
    // tile ahead (during this tile's offset loop)
    uint32_t mv_pf = 0;
    int q = DIRECT ? run0 + wi : (int)blockIdx.x;
    if constexpr (!DIRECT)
        if (q < p.ntiles) mv_pf = tile_mask(q, 0);
    constexpr int NX = C::NX;
    static_assert(NX <= 3, "index registers per lane");
    // lane l of wave w holds the caller index of slot 4 NW (16x + (l >> 2)) +
    // 4w + (l & 3) of a tile in d[x]
    auto dslot = [&](int x) -> int { return 4 * NW * (16 * x + (lane >> 2)) + 4 * wv + (lane & 3); };
    int32_t d_pf[NX];
    int pf_tile = -1;
    // the counter's old value (the next tile is gx + it), from the lead lane;
    // passed to every wave through LDS by the caller.  The counter's address
    // is offset by a register the compiler cannot see into, so that the
    // atomic is not rewritten as a wave-wide reduction whose broadcast would
    // wait for the result at once: the result is waited for where it is
    // used, after the staging's DMAs are issued.
    auto take_next = [&]() -> uint32_t {
        uint32_t v = 0;
        if (lead) {
            uint32_t z;
            asm volatile("v_mov_b32 %0, 0" : "=v"(z));
            v = atomicAdd(qctr + z, 1u);
        }
        return v;
    };

    while (DIRECT ? q < run1 : q < p.ntiles) {
        const int64_t tq = q;
        uint32_t mv_cur = 0;
        if constexpr (!DIRECT) mv_cur = mv_pf;
        if (p.dcount) {
            const uint32_t dcq = p.dcount[tq];
            if (DIRECT ? dcq != kNoDistinct : dcq == kNoDistinct) {   // uniform
                if constexpr (DIRECT) {
                    q += Wx;
                } else {
                    const uint32_t v = take_next();
                    if (lead) next_s = v + G;
                    __syncthreads();
                    q = (int)__builtin_amdgcn_readfirstlane(next_s);
                    __syncthreads();   // next_s is read
                    mv_pf = q < p.ntiles ? tile_mask(q, 0) : 0u;
                }
                continue;
            }
        }
        if constexpr (DIRECT) load_order(tq);
        // (the accumulators are cleared after the row copies are issued, so
        // that they hold no registers while the copies' addresses do)
        auto clear_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        };
        if constexpr (DIRECT) clear_acc();
        const int64_t row0 = tq * R;
        if constexpr (!DIRECT) {
            // The tile's distinct rows in one staging pass, or (past the
            // cap) in three, one per layer of nine offsets, each running its
            // layer's active offsets: every output still adds its terms in
            // ascending offset order.
            const uint32_t dcr = p.dcount[tq];
            const bool layered = (dcr & kLayerPasses) != 0u;   // uniform
            const uint32_t mv = mv_cur;
            const uint64_t act = __ballot(mv != 0u);
            const uint64_t act0 = layered ? act & 0x1FFull : act;
            sv_tile = tq;
            const uint32_t qn_v = take_next();   // in flight during the staging
            // The row copies of pass ps go out first: the first pass's indices
            // were requested with the previous tile's copies (else now, waited
            // for alone), and every other load of the pass is issued after
            // them, so that nothing waits for it before the copies are on
            // their way.  Four slots per DMA: DMA i (slots 4i .. 4i + 3) is
            // wave i % NW's.
            auto stage = [&](int ps) __attribute__((always_inline)) {
                const int dcp = layered ? layer_rows(dcr, ps) : (int)dcr;   // rows of this pass
                int32_t d[NX];
                if (ps == 0 && pf_tile == q) {
#pragma unroll
                    for (int x = 0; x < NX; ++x) d[x] = d_pf[x];
                } else {
                    const int32_t* dr = p.drow + tq * LCAP + CAP * ps;
#pragma unroll
                    for (int x = 0; x < NX; ++x) d[x] = dslot(x) < dcp ? dr[dslot(x)] : 0;
                    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the indices (only on this path)
                }
                // In batches of NBT DMAs: first every lane's source row of each
                // DMA of the batch (cross-lane reads), then the batch's DMAs back
                // to back (a wait for the LDS reads, not the DMAs: those count
                // as vector memory only).
                constexpr int NIW = (CAP / 4 + NW - 1) / NW;   // DMAs per wave at most
                constexpr int NBT = 5;
                static_assert(NIW <= 16 * NX && 4 * NW * NIW >= CAP && NIW % NBT == 0, "index registers");
                // slot sl = 4 (wv + NW jj) + (lane >> 4): its swizzle f(sl) = 2 ((sl >> 1)
                // & 7) depends on sl mod 16 only, i.e. (NW a multiple of 4) on wv and
                // the lane, so the source chunk is the same for all of the wave's DMAs
                static_assert(NW % 4 == 0, "one chunk swizzle per lane");
                const uint32_t c = (uint32_t)n16 ^ (2u * ((uint32_t)(2 * wv + (lane >> 5)) & 7u));
                const uint8_t* src_c = feats + 16 * c;
                // (lane 4 (jj & 15) + (lane >> 4) of d[jj >> 4]: one base address,
                // the rest in the permute's immediate offset)
                const int pba = 4 * (lane >> 4);
#pragma unroll
                for (int j0 = 0; j0 < NIW; j0 += NBT) {
                    int32_t rsrc[NBT];
#pragma unroll
                    for (int u = 0; u < NBT; ++u)
                        rsrc[u] = __builtin_amdgcn_ds_bpermute(pba + 16 * ((j0 + u) & 15), d[(j0 + u) >> 4]);
#pragma unroll
                    for (int u = 0; u < NBT; ++u) {
                        const int i = wv + NW * (j0 + u);
                        // slot 4 i + (lane >> 4) < dcp, with the bound kept scalar
                        // (else the per-DMA lane slots are precomputed for the whole
                        // kernel and spill)
                        if ((lane >> 4) < __builtin_amdgcn_readfirstlane(dcp - 4 * i))
                            __builtin_amdgcn_global_load_lds(
                                src_c + (size_t)(uint32_t)rsrc[u] * 256,
                                (__attribute__((address_space(3))) void*)(rows + (size_t)(4 * i) * 256), 16, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // the tile's slot codes (K x 256 bytes) into L2 for the offset
            // loop's per-offset loads: 256-byte DMAs into an area nobody reads
            // (BN = 64: surf1024 -2%; at BN = 128 no gain, and a spill)
            if constexpr (BN == 64) {
                const uint8_t* smb = (const uint8_t*)p.smap + (size_t)tq * K * (2 * R);
                for (int i = wv; i < K; i += NW)
                    __builtin_amdgcn_global_load_lds(smb + (2 * R) * i + 4 * lane,
                                                     (__attribute__((address_space(3))) void*)dump, 4, 0, 0);
            }
            stage(0);
            // the first active offset's slot codes and w (K <= 27: one run),
            // the output rows
            if (act0) {
                load_sv(__builtin_ctzll(act0), svb[0]);
                load_w(__builtin_ctzll(act0), wb[0]);
            }
            load_order(tq);
            if (lead) next_s = qn_v + G;
            clear_acc();
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0): the rows, next_s
            barrier_only();
            // the next tile's masks and row indices (next_s is next written
            // during the next tile's staging, after the epilogue's barriers)
            const int qn = (int)__builtin_amdgcn_readfirstlane(next_s);
            mv_pf = qn < p.ntiles ? tile_mask(qn, 0) : 0u;
            if (qn < p.ntiles) {
                const int32_t* drn = p.drow + (int64_t)qn * LCAP;
#pragma unroll
                for (int x = 0; x < NX; ++x) d_pf[x] = dslot(x) < CAP ? drn[dslot(x)] : 0;
                pf_tile = qn;
            }
            if (act0) run(act0, 0, mv, [](int i) { return i; }, true);
            if (layered) {
                // the other two layers (their first slot codes and w
                // requested after the barrier, with the accumulators live)
                for (int ps = 1; ps < kDistinctLayers; ++ps) {
                    sync_lds();   // every wave is past its last row read of the previous pass
                    stage(ps);
                    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the rows
                    barrier_only();
                    const uint64_t actp = act & (0x1FFull << (9 * ps));
                    if (actp) run(actp, 0, mv, [](int i) { return i; }, false);
                }
            }
            q = qn;
        } else {
            // offsets in windows of 32, active ones two at a time
            for (int kb = 0; kb < K; kb += 32) {
                const uint32_t mv = tile_mask(tq, kb);
                uint64_t act = __ballot(mv != 0u);
                while (act) {
                    const int ia = __builtin_ctzll(act);
                    act &= act - 1;
                    const bool hb = act != 0;
                    const int ib = hb ? __builtin_ctzll(act) : 0;
                    act &= act - 1;
                    uint64_t pair = (1ull << ia) | (hb ? (1ull << ib) : 0ull);
                    // stage the pair's rows: slot R c + r for row r of offset c
                    // of the pair; R / 4 DMAs of four rows per offset, R / 4 / NW
                    // per wave
                    constexpr int DPW = R / 4 / NW;
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        if (c == 1 && !hb) break;
                        const int k = kb + (c == 0 ? ia : ib);
                        const int32_t* nb = p.nbr_m + (int64_t)k * p.Npad + row0;
                        int32_t nv[DPW];
#pragma unroll
                        for (int x = 0; x < DPW; ++x) nv[x] = nb[4 * (wv + NW * x) + (lane >> 4)];
#pragma unroll
                        for (int x = 0; x < DPW; ++x) {
                            const int i = wv + NW * x;
                            const int s = R * c + 4 * i + (lane >> 4);
                            const uint32_t ch = (uint32_t)n16 ^ (2u * (((uint32_t)s >> 1) & 7u));
                            if ((uint32_t)nv[x] < N32)
                                __builtin_amdgcn_global_load_lds(
                                    feats + (size_t)(uint32_t)nv[x] * 256 + 16 * ch,
                                    (__attribute__((address_space(3))) void*)(rows + (size_t)(R * c + 4 * i) * 256), 16, 0,
                                    0);
                        }
                        // slot codes: thread t = row t
                        if (t < R) {
                            const int32_t m = nb[t];
                            const uint32_t code = (uint32_t)m < N32 ? slot_code((uint32_t)(R * c + t)) : slot_code(CAP);
                            *(uint16_t*)(sml + c * (2 * R) + slot_pos(t) * 2) = (uint16_t)code;
                        }
                    }
                    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the pair's rows
                    sync_lds();
                    const int iaa = ia;
                    run(pair, kb, mv, [iaa](int i) { return i == iaa ? 0 : 1; }, false);
                    sync_lds();   // the pair's rows are read
                }
            }
            q += Wx;
        }
        epilogue();
    }
    // this workgroup's last take (a tile past the end) is done: the last
    // workgroup of the channel group to get here clears the counters
    if constexpr (!DIRECT) {
        if (lead && atomicAdd(qctr + 1, 1u) == (uint32_t)G - 1u) {
            atomicExch(qctr, 0u);
            atomicExch(qctr + 1, 0u);
        }
    }
}

// ---------------------------------------------------------------------------
// Small fp32 maps: the offsets split over the waves of a workgroup.
//
// With few rows the fp32 kernel below runs few workgroups, each stepping
// through the active offsets one after another, so a launch lasts about K
// load latencies.  Here a workgroup takes NBS 16-row blocks of the schedule
// and kSplitBN output channels; wave v of its kSplitWaves takes the offsets k
// with k % kSplitWaves == v, ascending, skipping those no row of the
// workgroup has, and accumulates its own partial sums, with its operands
// loaded straight from global memory one offset ahead (the neighbour indices
// two ahead).  The partial sums are added through LDS in wave order, then the
// bias.  Which wave adds a term depends on its offset alone, and a missing
// neighbour adds exact zeros, so the result does not depend on which rows
// share a block.
// MFMA 16x16x4 fp32 with srcA = w (16 output channels): in k-step s, lane
// l = m + 16 g holds w[k][g NS + s][co0 + 2m + j] for tile j (srcA) and
// feats[nbr][g NS + s] of row m (srcB), so a lane's NS feature values are
// contiguous (NS / 4 16-byte loads) and its w values of both tiles are one
// 8-byte load; it ends with channels 8g .. 8g + 7 of row l & 15 (tile j
// holding the channels 8g + 2i + j).
// (For bf16, gathering each row once per offset and channel group costs more
// than the offset chain it removes; the bf16 kernel takes smaller tiles
// instead.)
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 8;
constexpr int kSplitBN = 32;
constexpr int64_t kSplitMaxN = 65536;   // up to this many rows the split kernel runs

template <int CI, int NBS>
__global__ void __launch_bounds__(64 * kSplitWaves) k_fwd_split(FwdParams p) {
    constexpr int NW = kSplitWaves, BN = kSplitBN, NJ = BN / 16;
    constexpr int NS = CI / 4;                 // MFMA k-steps per offset
    __shared__ __attribute__((aligned(16))) f32x4_t red[NW][NJ][64];
    __shared__ uint32_t bmask[kMaxK];         // bit b: block b of the workgroup has offset k

    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int g = lane >> 4, n16 = lane & 15;
    const int64_t row0 = (int64_t)blockIdx.x * (16 * NBS);
    const int co0 = (int)blockIdx.y * BN;
    const int K = p.K;
    const int Co = p.Co;
    const uint32_t N32 = (uint32_t)p.N;
    const float* __restrict__ feats = (const float*)p.feats;
    const float* __restrict__ w = (const float*)p.w;

    {
        static_assert(kTileRows % (16 * NBS) == 0, "blocks inside one tile");
        const int64_t tile = row0 / kTileRows;
        const int bit = (int)((row0 % kTileRows) / 16);
        for (int k = t; k < K; k += 64 * NW)
            bmask[k] = ((uint32_t)p.blkmask[tile * K + k] >> bit) & ((1u << NBS) - 1u);
    }
    __syncthreads();

    // this wave's offsets with some row present, ascending
    auto next_k = [&](int k) -> int {
        for (k += NW; k < K; k += NW)
            if (bmask[k]) return k;
        return K;
    };
    auto load_nbr = [&](int k, int32_t (&nb)[NBS]) {
#pragma unroll
        for (int b = 0; b < NBS; ++b)
            nb[b] = k < K ? p.nbr_m[(int64_t)k * p.Npad + row0 + 16 * b + n16] : (int32_t)N32;
    };
    static_assert(NJ == 2 && NS % 4 == 0, "tile pair, 16-byte row pieces");
    auto load_ops = [&](int k, const int32_t (&nb)[NBS], float (&a)[NS][NJ], float (&bf)[NBS][NS]) {
#pragma unroll
        for (int b = 0; b < NBS; ++b) {
            const bool ok = (uint32_t)nb[b] < N32;
            const float* src = feats + (int64_t)(ok ? nb[b] : 0) * CI + g * NS;
#pragma unroll
            for (int v = 0; v < NS / 4; ++v) {
                f32x4_t x = *(const f32x4_t*)(src + 4 * v);
                if (!ok) x = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) bf[b][4 * v + e] = x[e];
            }
        }
        const float* wk = w + (int64_t)k * CI * Co + (int64_t)(g * NS) * Co + co0 + 2 * n16;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x2_t x = *(const f32x2_t*)(wk + (int64_t)s * Co);
            a[s][0] = x[0];
            a[s][1] = x[1];
        }
    };

    f32x4_t acc[NBS][NJ];
#pragma unroll
    for (int b = 0; b < NBS; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float a[2][NS][NJ], bfr[2][NBS][NS];
    int32_t nb_next[NBS];
    int kc = wv < K && bmask[wv] ? wv : next_k(wv);
    int kn = kc < K ? next_k(kc) : K;
    if (kc < K) {
        int32_t nb0[NBS];
        load_nbr(kc, nb0);
        load_ops(kc, nb0, a[0], bfr[0]);
    }
    load_nbr(kn, nb_next);
    // offset kc from buffer P while offset kn loads into the other one
    // (buffers named at compile time, so that they stay in registers)
    auto step = [&](auto PC) -> bool {
        constexpr int P = decltype(PC)::value;
        if (kc >= K) return false;
        const int kn2 = kn < K ? next_k(kn) : K;
        int32_t nb2[NBS];
        load_nbr(kn2, nb2);
        if (kn < K) load_ops(kn, nb_next, a[P ^ 1], bfr[P ^ 1]);
        const uint32_t bm = bmask[kc];
#pragma unroll
        for (int b = 0; b < NBS; ++b) {
            if (!((bm >> b) & 1u)) continue;
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[P][s][j], bfr[P][b][s], acc[b][j], 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < NBS; ++b) nb_next[b] = nb2[b];
        kc = kn;
        kn = kn2;
        return true;
    };
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }

    // per block: the partial sums added in wave order, then the bias
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
        if (b) __syncthreads();   // the previous block's sums are read
#pragma unroll
        for (int j = 0; j < NJ; ++j) red[wv][j][lane] = acc[b][j];
        __syncthreads();
        if (t < 128) {
            // thread half h writes channels 8g + 4h .. + 3: elements 2h, 2h + 1 of both tiles
            const int h = t >> 6;
            f32x4_t s0 = red[0][0][lane], s1 = red[0][1][lane];
#pragma unroll
            for (int v = 1; v < NW; ++v) {
                s0 += red[v][0][lane];
                s1 += red[v][1][lane];
            }
            f32x4_t sum = h ? f32x4_t{s0[2], s1[2], s0[3], s1[3]} : f32x4_t{s0[0], s1[0], s0[1], s1[1]};
            const int c = co0 + 8 * g + 4 * h;
            if (p.bias) sum += f32x4_t{p.bias[c], p.bias[c + 1], p.bias[c + 2], p.bias[c + 3]};
            const int32_t n_out = p.order[row0 + 16 * b + n16];
            if (n_out >= 0) *(f32x4_t*)((float*)p.out + (int64_t)n_out * Co + c) = sum;
        }
    }
}

// blocks per workgroup: enough workgroups for two per CU where the map
// allows, at most 2 where four blocks' operands would not fit the registers
template <int CI>
hipError_t launch_split(const FwdParams& fp, int cus, hipStream_t s) {
    constexpr int MAXB = CI <= 32 ? 4 : 2;
    const int64_t nblk = fp.Npad / 16;
    const int64_t want = 2 * (int64_t)cus;
    int nbs = nblk >= 4 * want ? 4 : nblk >= 2 * want ? 2 : 1;
    if (nbs > MAXB) nbs = MAXB;
    const dim3 grid((unsigned)(nblk / nbs), (unsigned)(fp.Co / kSplitBN));
    const dim3 block(64 * kSplitWaves);
    if constexpr (MAXB == 4) {
        if (nbs == 4) {
            k_fwd_split<CI, 4><<<grid, block, 0, s>>>(fp);
            return hipGetLastError();
        }
    }
    if (nbs == 2) k_fwd_split<CI, 2><<<grid, block, 0, s>>>(fp);
    else k_fwd_split<CI, 1><<<grid, block, 0, s>>>(fp);
    return hipGetLastError();
}

// Staged w row pitch (floats) of the fp32 kernel: the rows read by lane
// groups g and g + 1 (CI / 4 rows apart) start 64 banks apart for CI = 32
// and 64, so each half-wave's 16-byte reads are free of bank conflicts.
template <int CI, int BN>
constexpr int f32_pitch() { return BN + (CI == 32 ? 8 : 4); }

// MFMA roles: srcA = gathered rows (M = 16 rows), srcB = w (N = 16 output
// channels), K = 4 input channels (lane group g takes ci = g CI/4 + s in
// k-step s).  Lane n of tile j holds channel co0 + NJ n + j, so a lane's
// srcB values of all NJ tiles are NJ consecutive floats of a staged w row
// (16-byte LDS reads) and its outputs NJ consecutive channels of a row
// (16-byte stores).
template <int CI, int BN, int NB, typename FT>
__global__ void __launch_bounds__(256) k_fwd_f32(FwdParams p) {
    typedef typename Gather4<FT>::raw Raw;
    constexpr int BM = 4 * NB * 16;
    constexpr int NA = CI / 4;                  // A values per lane per block (= MFMA k-steps)
    constexpr int NV = CI / 16;                 // float4 loads per lane per block
    constexpr int NJ = BN / 16;
    static_assert(NJ % 2 == 0, "channel pairs per lane");
    constexpr int PITCH = f32_pitch<CI, BN>();  // floats per staged w row
    constexpr int WCH = CI * BN / 4;            // float4 chunks of w[k][:, co0:co0+BN]
    constexpr int WPT = (WCH + 255) / 256;
    constexpr uint32_t TBITS = (1u << (4 * NB)) - 1u;

    __shared__ __attribute__((aligned(16))) float ws[2][CI * PITCH];
    __shared__ uint16_t tmask[kMaxK];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int tile = xcd_tile(blockIdx.x, p.ntiles);
    const int64_t row0 = (int64_t)tile * BM;
    const int co0 = blockIdx.y * BN;
    // block b of this wave is block wave + 4b of the tile (see the bf16 kernel)
    auto brow = [&](int b) -> int64_t { return row0 + (int64_t)(wave + b * 4) * 16; };
    const int K = p.K;
    const uint32_t N32 = (uint32_t)p.N;
    const FT* __restrict__ feats = (const FT*)p.feats;
    const float* __restrict__ w = (const float*)p.w;
    const int Co = p.Co;

    {
        const int64_t mt = row0 / kTileRows;
        const int msh = (int)((row0 % kTileRows) / 16);
        for (int k = t; k < K; k += 256)
            tmask[k] = (uint16_t)((p.blkmask[mt * K + k] >> msh) & TBITS);
    }
    __syncthreads();

    auto next_k = [&](int k) {
        for (++k; k < K; ++k)
            if (tmask[k]) return k;
        return K;
    };
    auto load_nbr = [&](int k) -> int32_t {
        if (lane < NB * 16) return p.nbr_m[(int64_t)k * p.Npad + brow(lane >> 4) + (lane & 15)];
        return (int32_t)N32;
    };
    auto gather = [&](int32_t nbv, Raw (&a)[NB][NV]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int32_t nb = __shfl(nbv, b * 16 + (lane & 15));
            const bool ok = (uint32_t)nb < N32;
            const FT* src = feats + (int64_t)(ok ? nb : 0) * CI + (lane >> 4) * NA;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                Raw x = *(const Raw*)(src + 4 * v);
                if (!ok) x = (Raw)0;
                a[b][v] = x;
            }
        }
    };
    auto convert = [&](const Raw (&r)[NB][NV], f32x4_t (&a)[NB][NV]) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < NV; ++v) a[b][v] = as_f32x4(r[b][v]);
    };
    auto load_w = [&](int k, f32x4_t (&wr)[WPT]) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = t + 256 * i;
            if (WCH % 256 == 0 || e < WCH) {
                const int ci = e / (BN / 4), c4 = e % (BN / 4);
                wr[i] = *(const f32x4_t*)(w + ((int64_t)k * CI + ci) * Co + co0 + c4 * 4);
            }
        }
    };
    auto store_w = [&](const f32x4_t (&wr)[WPT], float* dst) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = t + 256 * i;
            if (WCH % 256 == 0 || e < WCH) {
                const int ci = e / (BN / 4), c4 = e % (BN / 4);
                *(f32x4_t*)(dst + ci * PITCH + c4 * 4) = wr[i];
            }
        }
    };

    f32x4_t acc[NB][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    f32x4_t a_cur[NB][NV];
    Raw a_nxt[NB][NV];
    f32x4_t wr[WPT];

    int kc = tmask[0] ? 0 : next_k(0);
    if (kc < K) {
        const int32_t nbv = load_nbr(kc);
        load_w(kc, wr);
        gather(nbv, a_nxt);
        store_w(wr, ws[0]);
        convert(a_nxt, a_cur);
    }
    int kn = kc < K ? next_k(kc) : K;
    int32_t nbv_n = load_nbr(kn < K ? kn : (kc < K ? kc : 0));
    __syncthreads();

    int buf = 0;
    while (kc < K) {
        const int kn_eff = kn < K ? kn : kc;
        const int kn2 = kn < K ? next_k(kn) : K;
        gather(nbv_n, a_nxt);
        load_w(kn_eff, wr);
        const int32_t nbv_n2 = load_nbr(kn2 < K ? kn2 : kn_eff);

        const uint32_t tm = tmask[kc];
        uint32_t wb = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) wb |= ((tm >> (wave + b * 4)) & 1u) << b;
        if (wb) {
            const float* wsb = ws[buf];
#pragma unroll
            for (int s = 0; s < NA; ++s) {
                const int ci = (lane >> 4) * NA + s;
                const float* wrow = wsb + ci * PITCH + NJ * (lane & 15);
                float bw[NJ];
                if constexpr (NJ == 2) {
                    const f32x2_t x = *(const f32x2_t*)wrow;
                    bw[0] = x[0];
                    bw[1] = x[1];
                } else {
#pragma unroll
                    for (int v = 0; v < NJ / 4; ++v) {
                        const f32x4_t x = *(const f32x4_t*)(wrow + 4 * v);
#pragma unroll
                        for (int e = 0; e < 4; ++e) bw[4 * v + e] = x[e];
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (wb & (1u << b)) {
                        const float av = a_cur[b][s >> 2][s & 3];
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bw[j], acc[b][j],
                                                                            0, 0, 0);
                    }
                }
            }
        }
        if (kn < K) store_w(wr, ws[buf ^ 1]);
        __syncthreads();
        convert(a_nxt, a_cur);
        nbv_n = nbv_n2;
        kc = kn;
        kn = kn2;
        buf ^= 1;
    }

    // lane: rows brow(b) + 4g + i, channels co0 + NJ n16 .. + NJ - 1
    float* __restrict__ out = (float*)p.out;
    const int col0 = co0 + NJ * (lane & 15);
    float bsv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bsv[j] = p.bias ? p.bias[col0 + j] : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = brow(b) + 4 * (lane >> 4) + i;
            const int32_t n_out = p.order[r];
            if (n_out >= 0) {
                float* dst = out + (int64_t)n_out * Co + col0;
                if constexpr (NJ == 2) {
                    *(f32x2_t*)dst = f32x2_t{acc[b][0][i] + bsv[0], acc[b][1][i] + bsv[1]};
                } else {
#pragma unroll
                    for (int v = 0; v < NJ / 4; ++v)
                        *(f32x4_t*)(dst + 4 * v) = f32x4_t{acc[b][4 * v][i] + bsv[4 * v], acc[b][4 * v + 1][i] + bsv[4 * v + 1],
                                                           acc[b][4 * v + 2][i] + bsv[4 * v + 2], acc[b][4 * v + 3][i] + bsv[4 * v + 3]};
                }
            }
        }
    }
}

// blocks per wave for a (dtype, Ci): bounded by the A-fragment registers
constexpr int nb_for(int dtype, int ci) {
    return dtype == SPCONV_BF16 ? (ci <= 128 ? 4 : 2) : (ci <= 64 ? 2 : (ci == 128 ? 2 : 1));
}

// LDS bytes of the staged weights (two buffers) must fit gfx950's 160 KB.
template <int CI, int BN>
constexpr bool f32_fits() { return 2 * CI * f32_pitch<CI, BN>() * 4 + 2 * kMaxK <= 160 * 1024; }

// bf16 launch shape for (CI, BN): 16-row blocks per wave, waves (rows x
// channels) and gather look-ahead, bounded by registers and LDS.  Measured on
// the surface workloads: eight waves (two per SIMD) of 32 rows x BN channels,
// gathering one offset ahead, beat four waves of 64 rows (one per SIMD) by
// about 20%; a deeper look-ahead did not help.  One block per wave at Ci = 256
// keeps the feature stages in registers; so it does for float32 features
// (cast as they are gathered), whose raw stages take twice the registers.
template <int CI, int BN, typename FT>
struct Bf16Shape {
    static constexpr int NB = (CI <= 128 && sizeof(FT) == 2) ? 2 : 1, NWR = 8, NWC = 1, D = 1;
};

// Packs w[k][:, tile*BN : tile*BN + BN] into the staged plane layout of the
// LDS-staged kernels: unit (u, wrow(u, r)) of slice (k, tile), u =
// input-channel group of 8, r = 16j + m < BN, holds w[k][8u .. 8u+7][tile*BN
// + co(j, m)] with co(j, m) = (m >> 2) 4NJ + 4j + (m & 3).  The slice is
// w[k][:, tile] alone (CI * BN * 2 bytes).
template <int CI, int BN>
__global__ void __launch_bounds__(256) k_pack_w(const uint16_t* __restrict__ w, int K, int Co,
                                                u32x4_t* __restrict__ wpack) {
    constexpr int NJ = BN / 16, UNITS = (CI / 8) * BN;
    const int nct = Co / BN;
    const int64_t total = (int64_t)K * nct * UNITS;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t slice = e / UNITS;
        const int unit = (int)(e % UNITS);
        const int k = (int)(slice / nct), tile = (int)(slice % nct);
        const int u = unit / BN, r = wrow(u, unit % BN);
        const int j = r >> 4, m = r & 15;
        const int co = tile * BN + (m >> 2) * 4 * NJ + 4 * j + (m & 3);
        const uint16_t* src = w + ((int64_t)k * CI + 8 * u) * Co + co;
        uint16_t h[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) h[q] = src[(int64_t)q * Co];
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
        wpack[e] = v;
    }
}

// Packs w (K, 128, Co), Co % 64 == 0, into the fragment order of
// k_fwd_bf16_tile: 16-byte unit e = (((k NCG + cg) 4 + s) 4 + j) 64 + l
// (NCG = Co / 64, lane l = m + 16 g) holds w[k][32 s + 8 g .. + 7][64 cg +
// 16 (m >> 2) + 4 j + (m & 3)]: lane l's A operand of MFMA tile j, k-step s.
__global__ void __launch_bounds__(256) k_pack_w_frag(const uint16_t* __restrict__ w, int K, int Co,
                                                     u32x4_t* __restrict__ wpack) {
    const int NCG = Co / 64;
    const int64_t total = (int64_t)K * NCG * 16 * 64;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int l = (int)(e & 63), j = (int)((e >> 6) & 3), st = (int)((e >> 8) & 3);
        const int64_t rest = e >> 10;
        const int cg = (int)(rest % NCG), k = (int)(rest / NCG);
        const int m = l & 15, gg = l >> 4;
        const int co = 64 * cg + 16 * (m >> 2) + 4 * j + (m & 3);
        const uint16_t* src = w + ((int64_t)k * 128 + 32 * st + 8 * gg) * Co + co;
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (uint32_t)src[(int64_t)(2 * q) * Co] | ((uint32_t)src[(int64_t)(2 * q + 1) * Co] << 16);
        wpack[e] = v;
    }
}

// Ci = 128 with Co % 64 == 0 packs for the tile kernel
bool frag_packed(int Ci, int Co) { return Ci == 128 && Co % 64 == 0; }

template <int CI, int BN, int NB, int NWR>
constexpr int lds_bytes() {
    return (NWR == 8 ? 2 : 1) * (CI / 8) * BN * 16 + NWR * NB * (CI / 32) * kDmaPitch + 4 * kMaxK + 64 +
           4 * kMaxTPW * NWR * NB * 16 + 4 * BN;
}
template <int CI, int BN, int NB, int NWR>
constexpr bool lds_fits() { return lds_bytes<CI, BN, NB, NWR>() * (8 / NWR) <= 160 * 1024; }
// Tiles per workgroup: two measured 0.4% (surf256) and 2% (surf1024) faster
// than one; four gave no further gain.
constexpr int kLdsTPW = 2;
template <int CI>
constexpr int lds_nb() { return CI <= 128 ? 2 : 1; }

int cu_count();

template <int CI, int BN, typename FT>
void launch_bf16(const FwdParams& fp, hipStream_t s) {
    if (fp.Npad / kTileRows < cu_count()) {
        // fewer 256-row tiles than CUs: 64-row tiles, four times the
        // workgroups (shell64: 33 -> 23.5 us)
        constexpr int NB = 1, NWR = 4;
        FwdParams q = fp;
        q.ntiles = (int)(fp.Npad / (NWR * NB * 16));
        dim3 grid((unsigned)q.ntiles, (unsigned)(fp.Co / BN));
        k_fwd_bf16<CI, BN, NB, NWR, 1, 1, FT><<<grid, dim3(64 * NWR), 0, s>>>(q);
        return;
    }
    using S = Bf16Shape<CI, BN, FT>;
    constexpr int BM = S::NWR * S::NB * 16;
    FwdParams q = fp;
    q.ntiles = (int)(fp.Npad / BM);
    dim3 grid((unsigned)q.ntiles, (unsigned)(fp.Co / BN));
    k_fwd_bf16<CI, BN, S::NB, S::NWR, S::NWC, S::D, FT><<<grid, dim3(64 * S::NWR * S::NWC), 0, s>>>(q);
}

// Tile-queue counters of the tile kernel: kQueueSlots slots of a [next,
// done] pair, zero when the library is loaded and set back to zero by the
// launch that used them; a launch takes Co / BN consecutive slots.  Launches
// take slots in turn (per device), so two launches share counters only when
// kQueueSlots slots have been handed out in between while the first one still
// runs.  In host code `tile_queue` only names the symbol; its device address
// comes from hipGetSymbolAddress, once per device with that device current.
constexpr uint32_t kQueueSlots = 8192;
__device__ __align__(256) uint32_t tile_queue[2 * kQueueSlots];
constexpr int kQueueDevices = 64;
std::mutex g_queue_mu;
uint32_t* g_queue_ptr[kQueueDevices] = {};
uint32_t g_queue_next[kQueueDevices] = {};

hipError_t queue_slots(hipStream_t s, uint32_t n, uint32_t** out) {
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kQueueDevices || n == 0 || n > kQueueSlots) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(g_queue_mu);
    if (!g_queue_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(tile_queue));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_queue_ptr[dev] = (uint32_t*)ptr;
    }
    uint32_t first = g_queue_next[dev];
    if (first + n > kQueueSlots) first = 0;   // n consecutive slots
    g_queue_next[dev] = (first + n) % kQueueSlots;
    *out = g_queue_ptr[dev] + 2 * first;
    return hipSuccess;
}

int cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

// The tile kernel over the tiles whose distinct rows fit LDS, then its
// DIRECT instantiation over the others (when any tile is over the cap, when
// the map has no slot lists, or when that is not known on the host).  Two
// persistent workgroups per CU.
template <int BN>
hipError_t launch_tile(const FwdParams& fp, int64_t max_distinct, hipStream_t s) {
    FwdParams q = fp;
    q.ntiles = (int)(fp.Npad / TileCfg<BN>::R);
    const int slots = TileCfg<BN>::WGS * cu_count();
    const unsigned gx = (unsigned)(q.ntiles < slots ? q.ntiles : slots);
    const dim3 grid(gx, (unsigned)(fp.Co / BN));
    const bool lists = fp.dcount && fp.K <= kDistinctMaxK;
    if (lists) {
        const hipError_t eq = queue_slots(s, grid.y, &q.queue);
        if (eq != hipSuccess) return eq;
        k_fwd_bf16_tile<BN, false><<<grid, dim3(64 * TileCfg<BN>::NW), 0, s>>>(q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (max_distinct >= 0 && max_distinct <= kDistinctListCap) return hipSuccess;
    } else {
        q.dcount = nullptr;   // every tile is direct
    }
    k_fwd_bf16_tile<BN, true><<<grid, dim3(64 * TileCfg<BN>::NW), 0, s>>>(q);
    return hipGetLastError();
}

template <int CI, int BN>
hipError_t launch_ci_bn(const FwdParams& fp, int dtype, int fdtype, hipStream_t s, bool staged,
                        int64_t max_distinct) {
    constexpr int NWR = 8;
    if constexpr (CI % 128 == 0 && lds_fits<CI, BN, lds_nb<CI>(), NWR>()) {
        if (dtype == SPCONV_BF16 && staged) {
            constexpr int NB = lds_nb<CI>();
            constexpr int BM = NWR * NB * 16;
            FwdParams q = fp;
            q.ntiles = (int)(fp.Npad / BM);
            // consecutive tiles per workgroup, with the offset list of all of
            // them (one entry per tile and active offset) within kMaxK
            q.tpw = kMaxK / fp.K;
            q.tpw = q.tpw < 1 ? 1 : (q.tpw > kLdsTPW ? kLdsTPW : q.tpw);
            dim3 grid((unsigned)((q.ntiles + q.tpw - 1) / q.tpw), (unsigned)(fp.Co / BN));
            if (fp.wpack)
                k_fwd_bf16_lds<CI, BN, NB, NWR, true><<<grid, dim3(64 * NWR), 0, s>>>(q);
            else
                k_fwd_bf16_lds<CI, BN, NB, NWR, false><<<grid, dim3(64 * NWR), 0, s>>>(q);
            return hipGetLastError();
        }
    }
    if (dtype == SPCONV_BF16) {
        if (fdtype == SPCONV_F32)
            launch_bf16<CI, BN, float>(fp, s);
        else
            launch_bf16<CI, BN, uint16_t>(fp, s);
    } else {
        if constexpr (f32_fits<CI, BN>()) {
            constexpr int NB = nb_for(SPCONV_F32, CI);
            constexpr int BM = 4 * NB * 16;
            FwdParams q = fp;
            q.ntiles = (int)(fp.Npad / BM);
            dim3 grid((unsigned)q.ntiles, (unsigned)(fp.Co / BN));
            if (fdtype == SPCONV_BF16)
                k_fwd_f32<CI, BN, NB, uint16_t><<<grid, dim3(256), 0, s>>>(q);
            else
                k_fwd_f32<CI, BN, NB, float><<<grid, dim3(256), 0, s>>>(q);
        } else {
            return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int CI>
hipError_t launch_ci(const FwdParams& fp, int dtype, int fdtype, int bn, hipStream_t s, bool staged,
                     int64_t max_distinct) {
    switch (bn) {
        case 128: return launch_ci_bn<CI, 128>(fp, dtype, fdtype, s, staged, max_distinct);
        case 64: return launch_ci_bn<CI, 64>(fp, dtype, fdtype, s, staged, max_distinct);
        default: return launch_ci_bn<CI, 32>(fp, dtype, fdtype, s, staged, max_distinct);
    }
}

int pick_bn(int Co) { return (Co % 128 == 0) ? 128 : (Co % 64 == 0) ? 64 : 32; }

// output-channel tile of the LDS-staged kernel (Ci = 256 is LDS-bound to 64)
int lds_bn(int Ci, int Co) {
    const int bn = pick_bn(Co);
    return (Ci == 256 && bn == 128) ? 64 : bn;
}

template <int CI, int BN>
size_t pack_bytes_t(int K, int Co) {
    return (size_t)K * (size_t)(Co / BN) * CI * BN * 2;
}

template <int CI>
size_t pack_bytes_ci(int K, int Co) {
    switch (lds_bn(CI, Co)) {
        case 128: return pack_bytes_t<CI, 128>(K, Co);
        case 64: return pack_bytes_t<CI, 64>(K, Co);
        default: return pack_bytes_t<CI, 32>(K, Co);
    }
}

template <int CI, int BN>
hipError_t launch_pack_t(const void* w, int K, int Co, void* wpack, hipStream_t s) {
    const int64_t units = (int64_t)K * (Co / BN) * (CI / 8) * BN;
    const int64_t blocks = (units + 255) / 256;
    k_pack_w<CI, BN><<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>((const uint16_t*)w, K, Co,
                                                                               (u32x4_t*)wpack);
    return hipGetLastError();
}

template <int CI>
hipError_t launch_pack_ci(const void* w, int K, int Co, void* wpack, hipStream_t s) {
    switch (lds_bn(CI, Co)) {
        case 128: return launch_pack_t<CI, 128>(w, K, Co, wpack, s);
        case 64: return launch_pack_t<CI, 64>(w, K, Co, wpack, s);
        default: return launch_pack_t<CI, 32>(w, K, Co, wpack, s);
    }
}

}  // namespace

namespace {

// Weights of the input gradient: wt[k][co][ci] = w[K-1-k][ci][co].  A 32 x 32
// tile of one offset's (Ci, Co) matrix goes through LDS so that both the read
// of w and the write of wt are row-contiguous.  Element size 2 or 4 bytes.
template <typename T>
__global__ void __launch_bounds__(256) k_mirror_w(const T* __restrict__ w, int K, int Ci, int Co,
                                                  T* __restrict__ wt) {
    __shared__ T tile[32][33];
    const int k = blockIdx.z;
    const int ci0 = blockIdx.y * 32, co0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
    const T* src = w + (int64_t)(K - 1 - k) * Ci * Co;
    T* dst = wt + (int64_t)k * Co * Ci;
#pragma unroll
    for (int r = ty; r < 32; r += 8)
        if (ci0 + r < Ci && co0 + tx < Co) tile[r][tx] = src[(int64_t)(ci0 + r) * Co + co0 + tx];
    __syncthreads();
#pragma unroll
    for (int r = ty; r < 32; r += 8)
        if (co0 + r < Co && ci0 + tx < Ci) dst[(int64_t)(co0 + r) * Ci + ci0 + tx] = tile[tx][r];
}

}  // namespace

hipError_t launch_mirror_weights(const void* w, int K, int Ci, int Co, int dtype, void* wt, hipStream_t stream) {
    dim3 grid((unsigned)((Co + 31) / 32), (unsigned)((Ci + 31) / 32), (unsigned)K);
    if (dtype == SPCONV_BF16)
        k_mirror_w<uint16_t><<<grid, dim3(256), 0, stream>>>((const uint16_t*)w, K, Ci, Co, (uint16_t*)wt);
    else
        k_mirror_w<float><<<grid, dim3(256), 0, stream>>>((const float*)w, K, Ci, Co, (float*)wt);
    return hipGetLastError();
}

size_t packed_weight_bytes(int K, int Ci, int Co, int dtype) {
    if (dtype != SPCONV_BF16 || !forward_supported(dtype, Ci, Co)) return 0;
    if (Ci == 128) return pack_bytes_ci<128>(K, Co);
    if (Ci == 256) return pack_bytes_ci<256>(K, Co);
    return 0;
}

hipError_t launch_pack_weights(const void* w, int K, int Ci, int Co, int dtype, void* wpack, hipStream_t stream) {
    if (packed_weight_bytes(K, Ci, Co, dtype) == 0) return hipSuccess;
    if (frag_packed(Ci, Co)) {
        const int64_t units = (int64_t)K * (Co / 64) * 16 * 64;
        const int64_t blocks = (units + 255) / 256;
        k_pack_w_frag<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>((const uint16_t*)w, K, Co,
                                                                                     (u32x4_t*)wpack);
        return hipGetLastError();
    }
    return Ci == 128 ? launch_pack_ci<128>(w, K, Co, wpack, stream) : launch_pack_ci<256>(w, K, Co, wpack, stream);
}

bool tile_forward(int dtype, int feats_dtype, int Ci, int Co) {
    return dtype == SPCONV_BF16 && feats_dtype == SPCONV_BF16 && Ci == 128 && Co % 64 == 0;
}

bool forward_supported(int dtype, int Ci, int Co) {
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16) return false;
    if (Ci != 32 && Ci != 64 && Ci != 128 && Ci != 256) return false;
    return Co >= 32 && Co <= 4096 && Co % 32 == 0;
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
    if (!forward_supported(a.dtype, a.Ci, a.Co) || a.K > kMaxK) return hipErrorInvalidValue;
    if (a.feats_dtype != SPCONV_F32 && a.feats_dtype != SPCONV_BF16) return hipErrorInvalidValue;
    if (a.cast_ws && a.feats_dtype == SPCONV_F32 && a.dtype == SPCONV_BF16) {
        // cast pass into the workspace, then the same-dtype forward on it
        const int64_t n8 = a.N * a.Ci / 8;
        const int64_t blocks = (n8 + 255) / 256;
        k_cast_bf16<<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, stream>>>(
            (const u32x4_t*)a.feats, (u32x4_t*)a.cast_ws, n8);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ForwardArgs b = a;
        b.feats = a.cast_ws;
        b.feats_dtype = SPCONV_BF16;
        b.cast_ws = nullptr;
        return launch_forward(b, stream);
    }
    FwdParams fp;
    fp.feats = a.feats;
    fp.nbr_m = a.nbr_m;
    fp.order = a.order;
    fp.blkmask = a.blkmask;
    fp.dcount = a.dcount;
    fp.drow = a.drow;
    fp.smap = a.smap;
    fp.w = a.w;
    fp.wpack = nullptr;
    fp.bias = a.bias;
    fp.out = a.out;
    fp.N = a.N;
    fp.Npad = a.Npad;
    fp.K = a.K;
    fp.Co = a.Co;
    fp.ntiles = 0;
    fp.tpw = 1;
    fp.queue = nullptr;
    int bn = pick_bn(a.Co);
    // small fp32 maps (fp32 features, Ci <= 64): the offsets of each 16-row
    // block split over the waves
    if (a.dtype == SPCONV_F32 && a.feats_dtype == SPCONV_F32 && a.N <= kSplitMaxN && a.Ci <= 64 &&
        a.Co % kSplitBN == 0)
        return a.Ci == 32 ? launch_split<32>(fp, cu_count(), stream) : launch_split<64>(fp, cu_count(), stream);
    // bf16, Ci = 128, Co % 64 == 0 with packed w: the tile kernel (64-bit
    // row addresses, any N)
    if (tile_forward(a.dtype, a.feats_dtype, a.Ci, a.Co) && a.wpack) {
        fp.wpack = a.wpack;
        return a.Co % 128 == 0 ? launch_tile<128>(fp, a.max_distinct, stream) : launch_tile<64>(fp, a.max_distinct, stream);
    }
    // The LDS-staged bf16 kernel addresses feats with 32-bit byte offsets.
    const bool staged = a.dtype == SPCONV_BF16 && a.feats_dtype == SPCONV_BF16 && a.Ci % 128 == 0 &&
                        (uint64_t)a.N * (uint64_t)a.Ci * 2u < (1ull << 32);
    if (staged) {
        bn = lds_bn(a.Ci, a.Co);
        fp.wpack = a.wpack;   // used by the staged kernel only
    }
    // fp32: 64-channel column tiles and (Ci <= 64) two blocks per wave keep the
    // kernel at three waves per SIMD; at surf512d2 (32 -> 256, dilation 2)
    // 128-channel tiles of four blocks per wave (one wave per SIMD) took
    // 5.62 ms, this shape 3.80 ms
    if (a.dtype == SPCONV_F32 && bn == 128) bn = 64;
    switch (a.Ci) {
        case 32: return launch_ci<32>(fp, a.dtype, a.feats_dtype, bn, stream, staged, a.max_distinct);
        case 64: return launch_ci<64>(fp, a.dtype, a.feats_dtype, bn, stream, staged, a.max_distinct);
        case 128: return launch_ci<128>(fp, a.dtype, a.feats_dtype, bn, stream, staged, a.max_distinct);
        default: return launch_ci<256>(fp, a.dtype, a.feats_dtype, bn, stream, staged, a.max_distinct);
    }
}

size_t cast_workspace_bytes(int64_t N, int Ci, int feats_dtype, int dtype) {
    return (feats_dtype == SPCONV_F32 && dtype == SPCONV_BF16) ? align_up((size_t)N * Ci * 2, 256) : 0;
}

}  // namespace spc
