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
// No atomics: every output element is written once by one lane, so results
// are deterministic.
#include "spconv_internal.h"

namespace spc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxK = 1024;

struct FwdParams {
    const void* feats;
    const int32_t* nbr_m;
    const int32_t* order;
    const uint16_t* blkmask;
    const void* w;
    const float* bias;
    void* out;
    int64_t N, Npad;
    int K, Co, ntiles;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
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

template <int CI, int BN, int NB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_fwd_bf16(FwdParams p) {
    constexpr int BM = 4 * NB * 16;
    constexpr int NS = CI / 32;                 // MFMA k-steps (32 ci each)
    constexpr int NJ = BN / 16;                 // 16-column MFMA tiles
    constexpr int CH = CI / 8;                  // 16-byte chunks per staged row
    constexpr int CMASK = (CH >= 8 ? 8 : CH) - 1;
    constexpr int WCH = CI * BN / 8;            // 16-byte chunks of w[k][:, co0:co0+BN]
    constexpr int WPT = (WCH + 255) / 256;
    constexpr uint32_t TBITS = (1u << (4 * NB)) - 1u;

    __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN * CI];
    __shared__ uint16_t tmask[kMaxK];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int tile = xcd_tile(blockIdx.x, p.ntiles);
    const int64_t row0 = (int64_t)tile * BM;
    const int co0 = blockIdx.y * BN;
    const int64_t wrow0 = row0 + wave * NB * 16;
    const int K = p.K;
    const uint32_t N32 = (uint32_t)p.N;
    const uint16_t* __restrict__ feats = (const uint16_t*)p.feats;
    const uint16_t* __restrict__ w = (const uint16_t*)p.w;
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
        if (lane < NB * 16) return p.nbr_m[(int64_t)k * p.Npad + wrow0 + lane];
        return (int32_t)N32;
    };
    auto gather = [&](int32_t nbv, bf16x8_t (&a)[NB][NS]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int32_t nb = __shfl(nbv, b * 16 + (lane & 15));
            const bool ok = (uint32_t)nb < N32;
            const uint16_t* src = feats + (int64_t)(ok ? nb : 0) * CI + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                u32x4_t v = *(const u32x4_t*)(src + 32 * s);
                if (!ok) v = u32x4_t{0u, 0u, 0u, 0u};
                a[b][s] = __builtin_bit_cast(bf16x8_t, v);
            }
        }
    };
    auto load_w = [&](int k, u32x4_t (&wr)[WPT]) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = t + 256 * i;
            if (WCH % 256 == 0 || e < WCH) {
                const int ci = (e & 7) + 8 * (e / BN);
                const int c8 = (e >> 3) % (BN / 8);
                wr[i] = *(const u32x4_t*)(w + ((int64_t)k * CI + ci) * Co + co0 + c8 * 8);
            }
        }
    };
    auto store_w = [&](const u32x4_t (&wr)[WPT], uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = t + 256 * i;
            if (WCH % 256 == 0 || e < WCH) {
                const int ci = (e & 7) + 8 * (e / BN);
                const int c8 = (e >> 3) % (BN / 8);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int n = c8 * 8 + jj;
                    const uint32_t word = wr[i][jj >> 1];
                    const uint16_t h = (uint16_t)((jj & 1) ? (word >> 16) : (word & 0xffffu));
                    dst[n * CI + (((ci >> 3) ^ (swz(n) & CMASK)) << 3) + (ci & 7)] = h;
                }
            }
        }
    };

    f32x4_t acc[NB][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    bf16x8_t a_cur[NB][NS], a_nxt[NB][NS];
    u32x4_t wr[WPT];

    int kc = tmask[0] ? 0 : next_k(0);
    if (kc < K) {
        const int32_t nbv = load_nbr(kc);
        load_w(kc, wr);
        gather(nbv, a_cur);
        store_w(wr, ws[0]);
    }
    int kn = kc < K ? next_k(kc) : K;
    int32_t nbv_n = load_nbr(kn < K ? kn : (kc < K ? kc : 0));
    __syncthreads();

    int buf = 0;
    while (kc < K) {
        const int kn_eff = kn < K ? kn : kc;          // loads stay unconditional
        const int kn2 = kn < K ? next_k(kn) : K;
        gather(nbv_n, a_nxt);
        load_w(kn_eff, wr);
        const int32_t nbv_n2 = load_nbr(kn2 < K ? kn2 : kn_eff);

        const uint32_t wb = (tmask[kc] >> (wave * NB)) & ((1u << NB) - 1u);
        if (wb) {
            const uint16_t* wsb = ws[buf];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8_t bw[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int n = j * 16 + (lane & 15);
                    const int chunk = 4 * s + (lane >> 4);
                    bw[j] = *(const bf16x8_t*)(wsb + n * CI + ((chunk ^ (swz(n) & CMASK)) << 3));
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (wb & (1u << b)) {
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_cur[b][s], bw[j],
                                                                                acc[b][j], 0, 0, 0);
                    }
                }
            }
        }
        if (kn < K) store_w(wr, ws[buf ^ 1]);
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < NS; ++s) a_cur[b][s] = a_nxt[b][s];
        nbv_n = nbv_n2;
        kc = kn;
        kn = kn2;
        buf ^= 1;
    }

    // epilogue: + bias, one RNE rounding, scatter rows to caller order
    uint16_t* __restrict__ out = (uint16_t*)p.out;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = wrow0 + b * 16 + 4 * (lane >> 4) + i;
            const int32_t n_out = p.order[r];
            if (n_out >= 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int col = co0 + j * 16 + (lane & 15);
                    const float v = acc[b][j][i] + (p.bias ? p.bias[col] : 0.f);
                    out[(int64_t)n_out * Co + col] = f32_to_bf16_rne(v);
                }
            }
        }
    }
}

template <int CI, int BN, int NB>
__global__ void __launch_bounds__(256) k_fwd_f32(FwdParams p) {
    constexpr int BM = 4 * NB * 16;
    constexpr int NA = CI / 4;                  // A values per lane per block (= MFMA k-steps)
    constexpr int NV = CI / 16;                 // float4 loads per lane per block
    constexpr int NJ = BN / 16;
    constexpr int PITCH = BN + 4;               // floats per staged w row
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
    const int64_t wrow0 = row0 + wave * NB * 16;
    const int K = p.K;
    const uint32_t N32 = (uint32_t)p.N;
    const float* __restrict__ feats = (const float*)p.feats;
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
        if (lane < NB * 16) return p.nbr_m[(int64_t)k * p.Npad + wrow0 + lane];
        return (int32_t)N32;
    };
    auto gather = [&](int32_t nbv, f32x4_t (&a)[NB][NV]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int32_t nb = __shfl(nbv, b * 16 + (lane & 15));
            const bool ok = (uint32_t)nb < N32;
            const float* src = feats + (int64_t)(ok ? nb : 0) * CI + (lane >> 4) * NA;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                f32x4_t x = *(const f32x4_t*)(src + 4 * v);
                if (!ok) x = f32x4_t{0.f, 0.f, 0.f, 0.f};
                a[b][v] = x;
            }
        }
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

    f32x4_t a_cur[NB][NV], a_nxt[NB][NV];
    f32x4_t wr[WPT];

    int kc = tmask[0] ? 0 : next_k(0);
    if (kc < K) {
        const int32_t nbv = load_nbr(kc);
        load_w(kc, wr);
        gather(nbv, a_cur);
        store_w(wr, ws[0]);
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

        const uint32_t wb = (tmask[kc] >> (wave * NB)) & ((1u << NB) - 1u);
        if (wb) {
            const float* wsb = ws[buf];
#pragma unroll
            for (int s = 0; s < NA; ++s) {
                const int ci = (lane >> 4) * NA + s;
                float bw[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) bw[j] = wsb[ci * PITCH + j * 16 + (lane & 15)];
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
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < NV; ++v) a_cur[b][v] = a_nxt[b][v];
        nbv_n = nbv_n2;
        kc = kn;
        kn = kn2;
        buf ^= 1;
    }

    float* __restrict__ out = (float*)p.out;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = wrow0 + b * 16 + 4 * (lane >> 4) + i;
            const int32_t n_out = p.order[r];
            if (n_out >= 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int col = co0 + j * 16 + (lane & 15);
                    out[(int64_t)n_out * Co + col] = acc[b][j][i] + (p.bias ? p.bias[col] : 0.f);
                }
            }
        }
    }
}

// blocks per wave for a (dtype, Ci): bounded by the A-fragment registers
constexpr int nb_for(int dtype, int ci) {
    return dtype == SPCONV_BF16 ? (ci <= 128 ? 4 : 2) : (ci <= 64 ? 4 : (ci == 128 ? 2 : 1));
}

// LDS bytes of the staged weights (two buffers) must fit gfx950's 160 KB.
template <int CI, int BN>
constexpr bool f32_fits() { return 2 * CI * (BN + 4) * 4 + 2 * kMaxK <= 160 * 1024; }

template <int CI, int BN>
hipError_t launch_ci_bn(const FwdParams& fp, int dtype, hipStream_t s) {
    if (dtype == SPCONV_BF16) {
        constexpr int NB = nb_for(SPCONV_BF16, CI);
        constexpr int BM = 4 * NB * 16;
        FwdParams q = fp;
        q.ntiles = (int)(fp.Npad / BM);
        dim3 grid((unsigned)q.ntiles, (unsigned)(fp.Co / BN));
        k_fwd_bf16<CI, BN, NB><<<grid, dim3(256), 0, s>>>(q);
    } else {
        if constexpr (f32_fits<CI, BN>()) {
            constexpr int NB = nb_for(SPCONV_F32, CI);
            constexpr int BM = 4 * NB * 16;
            FwdParams q = fp;
            q.ntiles = (int)(fp.Npad / BM);
            dim3 grid((unsigned)q.ntiles, (unsigned)(fp.Co / BN));
            k_fwd_f32<CI, BN, NB><<<grid, dim3(256), 0, s>>>(q);
        } else {
            return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int CI>
hipError_t launch_ci(const FwdParams& fp, int dtype, int bn, hipStream_t s) {
    switch (bn) {
        case 128: return launch_ci_bn<CI, 128>(fp, dtype, s);
        case 64: return launch_ci_bn<CI, 64>(fp, dtype, s);
        default: return launch_ci_bn<CI, 32>(fp, dtype, s);
    }
}

int pick_bn(int Co) { return (Co % 128 == 0) ? 128 : (Co % 64 == 0) ? 64 : 32; }

}  // namespace

bool forward_supported(int dtype, int Ci, int Co) {
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16) return false;
    if (Ci != 32 && Ci != 64 && Ci != 128 && Ci != 256) return false;
    return Co >= 32 && Co <= 4096 && Co % 32 == 0;
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
    if (!forward_supported(a.dtype, a.Ci, a.Co) || a.K > kMaxK) return hipErrorInvalidValue;
    FwdParams fp;
    fp.feats = a.feats;
    fp.nbr_m = a.nbr_m;
    fp.order = a.order;
    fp.blkmask = a.blkmask;
    fp.w = a.w;
    fp.bias = a.bias;
    fp.out = a.out;
    fp.N = a.N;
    fp.Npad = a.Npad;
    fp.K = a.K;
    fp.Co = a.Co;
    fp.ntiles = 0;
    int bn = pick_bn(a.Co);
    if (a.dtype == SPCONV_F32 && a.Ci == 256 && bn == 128) bn = 64;  // LDS limit
    switch (a.Ci) {
        case 32: return launch_ci<32>(fp, a.dtype, bn, stream);
        case 64: return launch_ci<64>(fp, a.dtype, bn, stream);
        case 128: return launch_ci<128>(fp, a.dtype, bn, stream);
        default: return launch_ci<256>(fp, a.dtype, bn, stream);
    }
}

}  // namespace spc
