// Neighbour-map builder for gfx950.
//
// The page ("mlx_backend/sparse_conv_metal.py", `sparse_conv_metal` wrapper
// docstring) takes the (K, N) int32 map, sentinel N, as an input and does not
// show how it is made.  This builder produces it on the GPU:
//
//   1. pack:   range-check each coordinate, compute its 63-bit Morton code and
//              insert (coordinate key -> caller index) into an open-addressing
//              hash table (64-bit compare-and-swap, linear probing, load <= 1/2);
//              a second insert of the same key flags a duplicate.
//   2. sort:   LSD radix sort of (Morton code, caller index) on the bits that
//              vary across the set (8 bits per pass) -> voxels in Morton order.
//   3. query:  one workgroup per 256-row tile of the Morton order probes the
//              table for the K neighbours of each row, sorts the tile's rows by
//              their K-bit validity mask (rows with equal patterns end up in
//              the same 16-row blocks, so more blocks are entirely missing for
//              a given offset and the forward can skip them), then writes the
//              map in that row order plus one 16-bit block mask per (tile, k).
//
// All writes are plain vector stores and vector atomics.
#include "spconv_internal.h"

namespace spc {

namespace {

__device__ __forceinline__ bool coord_ok(int v) { return v >= -kCoordBias && v < kCoordBias; }

__device__ __forceinline__ unsigned long long coord_key(int x, int y, int z) {
    return ((unsigned long long)(uint32_t)(x + kCoordBias) << 42) |
           ((unsigned long long)(uint32_t)(y + kCoordBias) << 21) |
           (unsigned long long)(uint32_t)(z + kCoordBias);
}

// Spread the low 21 bits of v so that bit b lands on bit 3b (the usual
// shift-and-mask interleave).
__device__ __forceinline__ uint64_t spread3(uint32_t v) {
    uint64_t x = v & 0x1fffffu;
    x = (x | (x << 32)) & 0x001f00000000ffffull;
    x = (x | (x << 16)) & 0x001f0000ff0000ffull;
    x = (x | (x << 8)) & 0x100f00f00f00f00full;
    x = (x | (x << 4)) & 0x10c30c30c30c30c3ull;
    x = (x | (x << 2)) & 0x1249249249249249ull;
    return x;
}

// Morton code of biased coordinates: bit 3b = z_b, 3b+1 = y_b, 3b+2 = x_b.
__device__ __forceinline__ uint64_t morton3(int x, int y, int z) {
    return spread3((uint32_t)(z + kCoordBias)) | (spread3((uint32_t)(y + kCoordBias)) << 1) |
           (spread3((uint32_t)(x + kCoordBias)) << 2);
}

__device__ __forceinline__ uint32_t hash_slot(unsigned long long key, int log2_cap) {
    return (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> (64 - log2_cap));
}

__device__ __forceinline__ uint64_t wave_or(uint64_t v) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    for (int o = 32; o > 0; o >>= 1) {
        lo |= __shfl_xor(lo, o);
        hi |= __shfl_xor(hi, o);
    }
    return ((uint64_t)hi << 32) | lo;
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

__global__ void __launch_bounds__(256) k_pack_insert(const int32_t* __restrict__ coords, int64_t N,
                                                     uint64_t* __restrict__ codes,
                                                     uint32_t* __restrict__ idx, HashSlot* table,
                                                     int log2_cap, BuildFlags* flags) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint64_t diff = 0;
    if (i < N) {
        int x = coords[3 * i], y = coords[3 * i + 1], z = coords[3 * i + 2];
        idx[i] = (uint32_t)i;
        if (!coord_ok(x) || !coord_ok(y) || !coord_ok(z)) {
            atomicOr(&flags->range_error, 1u);
            codes[i] = 0;
        } else {
            uint64_t code = morton3(x, y, z);
            codes[i] = code;
            int x0 = coords[0], y0 = coords[1], z0 = coords[2];
            diff = code ^ morton3(x0, y0, z0);
            unsigned long long key = coord_key(x, y, z);
            const uint32_t mask = (1u << log2_cap) - 1u;
            uint32_t s = hash_slot(key, log2_cap);
            for (;;) {  // terminates: capacity >= 2N leaves empty slots
                unsigned long long prev = atomicCAS(&table[s].key, kEmptyKey, key);
                if (prev == kEmptyKey) {
                    table[s].val = (int32_t)i;
                    break;
                }
                if (prev == key) {
                    atomicOr(&flags->duplicate, 1u);
                    break;
                }
                s = (s + 1) & mask;
            }
        }
    }
    diff = wave_or(diff);
    if ((threadIdx.x & 63) == 0 && diff)
        atomicOr((unsigned long long*)&flags->morton_xor_or, (unsigned long long)diff);
}

// ---------------------------------------------------------------------------
// LSD radix sort, 8-bit digits.  Block b owns elements [b*4096, (b+1)*4096);
// within a block, element order is (round r, thread t) = b*4096 + r*256 + t,
// which is the input order, so each pass is stable.
// hist layout: hist[d * nblk + b] (digit-major).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kSortThreads) k_radix_hist(const uint64_t* __restrict__ codes,
                                                             int64_t N, int shift,
                                                             uint32_t* __restrict__ hist,
                                                             int64_t nblk) {
    __shared__ uint32_t h[kRadix];
    const int t = threadIdx.x;
    h[t] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortChunk;
#pragma unroll 4
    for (int r = 0; r < kSortItems; ++r) {
        int64_t e = base + (int64_t)r * kSortThreads + t;
        if (e < N) atomicAdd(&h[(uint32_t)(codes[e] >> shift) & (kRadix - 1)], 1u);
    }
    __syncthreads();
    hist[(int64_t)t * nblk + blockIdx.x] = h[t];
}

// Exclusive scan of each digit's row hist[d*nblk .. d*nblk+nblk) in place;
// totals[d] = the row's sum.  One block per digit.
__global__ void __launch_bounds__(256) k_radix_rowscan(uint32_t* __restrict__ hist, int64_t nblk,
                                                       uint32_t* __restrict__ totals) {
    __shared__ uint32_t part[256];
    const int t = threadIdx.x;
    uint32_t* row = hist + (int64_t)blockIdx.x * nblk;
    const int64_t per = (nblk + 255) / 256;
    const int64_t beg = t * per;
    const int64_t end = beg + per < nblk ? beg + per : nblk;
    uint32_t s = 0;
    for (int64_t i = beg; i < end; ++i) s += row[i];
    part[t] = s;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive Hillis-Steele scan
        uint32_t v = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t run = part[t] - s;
    for (int64_t i = beg; i < end; ++i) {
        uint32_t v = row[i];
        row[i] = run;
        run += v;
    }
    if (t == 255) totals[blockIdx.x] = part[255];
}

__global__ void __launch_bounds__(kSortThreads) k_radix_scatter(
    const uint64_t* __restrict__ codes_in, const uint32_t* __restrict__ idx_in, int64_t N, int shift,
    const uint32_t* __restrict__ hist, int64_t nblk, const uint32_t* __restrict__ totals,
    uint64_t* __restrict__ codes_out, uint32_t* __restrict__ idx_out) {
    __shared__ uint32_t base[kRadix];
    __shared__ uint32_t wcnt[kSortThreads / 64][kRadix];
    __shared__ uint32_t scan[kRadix];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = t >> 6;
    // digit start = exclusive scan of the totals, plus this block's row prefix
    uint32_t tot = totals[t];
    scan[t] = tot;
    __syncthreads();
    for (int o = 1; o < kRadix; o <<= 1) {
        uint32_t v = t >= o ? scan[t - o] : 0;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    base[t] = scan[t] - tot + hist[(int64_t)t * nblk + blockIdx.x];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t b0 = (int64_t)blockIdx.x * kSortChunk;
    for (int r = 0; r < kSortItems; ++r) {
        for (int w = 0; w < kSortThreads / 64; ++w) wcnt[w][t] = 0;
        __syncthreads();
        const int64_t e = b0 + (int64_t)r * kSortThreads + t;
        const bool act = e < N;
        uint64_t code = act ? codes_in[e] : 0;
        uint32_t id = act ? idx_in[e] : 0;
        uint32_t d = (uint32_t)(code >> shift) & (kRadix - 1);
        uint64_t peers = __ballot(act);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            bool bit = (d >> b) & 1u;
            uint64_t bal = __ballot(act && bit);
            peers &= bit ? bal : ~bal;
        }
        const uint32_t below = __popcll(peers & lt_mask);
        if (act && below == 0) wcnt[wv][d] = __popcll(peers);
        __syncthreads();
        if (act) {
            uint32_t pos = base[d] + below;
            for (int w = 0; w < wv; ++w) pos += wcnt[w][d];
            codes_out[pos] = code;
            idx_out[pos] = id;
        }
        __syncthreads();
        uint32_t add = 0;
        for (int w = 0; w < kSortThreads / 64; ++w) add += wcnt[w][t];
        base[t] += add;
        // the next round's clear is separated from these reads by the barrier
        // that follows it only after every thread has passed this point
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Tile query.  Block = one 256-row tile of the schedule, thread t = row t.
// mode 0: rows are Morton-sorted voxels, neighbours found in the hash table.
// mode 1: rows are caller rows, neighbours read from a caller-made map.
// ---------------------------------------------------------------------------
constexpr int kLdsK = 32;  // offsets kept in LDS; larger K probes twice

struct QueryArgs {
    const int32_t* coords;
    const uint32_t* morton_idx;   // mode 0
    const HashSlot* table;        // mode 0
    const int32_t* nbr_in;        // mode 1, (K, N)
    int64_t N, Npad;
    int K, side, dilation, log2_cap, mode;
    int32_t* nbr_m;
    int32_t* order;
    uint16_t* blkmask;
    MapInfo* info;
};

__device__ __forceinline__ int32_t probe(const QueryArgs& a, int64_t n, int cx, int cy, int cz, int k) {
    const int N32 = (int)a.N;
    if (a.mode == 1) {
        int32_t v = a.nbr_in[(int64_t)k * a.N + n];
        return ((uint32_t)v < (uint32_t)N32) ? v : N32;
    }
    const int s = a.side, r = (a.side - 1) >> 1;
    const int dc = k % s, db = (k / s) % s, da = k / (s * s);
    const int x = cx + a.dilation * (da - r);
    const int y = cy + a.dilation * (db - r);
    const int z = cz + a.dilation * (dc - r);
    if (!coord_ok(x) || !coord_ok(y) || !coord_ok(z)) return N32;
    const unsigned long long key = coord_key(x, y, z);
    const uint32_t mask = (1u << a.log2_cap) - 1u;
    uint32_t slot = hash_slot(key, a.log2_cap);
    for (;;) {
        const unsigned long long kk = a.table[slot].key;
        if (kk == key) return a.table[slot].val;
        if (kk == kEmptyKey) return N32;
        slot = (slot + 1) & mask;
    }
}

__global__ void __launch_bounds__(kTileRows) k_tile_query(QueryArgs a) {
    __shared__ int32_t nbs[kLdsK][kTileRows];
    __shared__ unsigned long long keys[kTileRows];
    __shared__ int32_t rowsrc[kTileRows];     // sorted position -> original thread
    __shared__ int32_t caller[kTileRows];     // original thread -> caller index (-1 pad)
    __shared__ int cx_s[kTileRows], cy_s[kTileRows], cz_s[kTileRows];
    __shared__ uint8_t wbits[kLdsK * 0 + 256][4];
    __shared__ unsigned long long cnt_s[4];

    const int t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int64_t tile = blockIdx.x;
    const int64_t j = tile * kTileRows + t;
    const int K = a.K;
    const int N32 = (int)a.N;

    int64_t n = -1;
    int cx = 0, cy = 0, cz = 0;
    if (j < a.N) {
        n = (a.mode == 0) ? (int64_t)a.morton_idx[j] : j;
        if (a.mode == 0) {
            cx = a.coords[3 * n];
            cy = a.coords[3 * n + 1];
            cz = a.coords[3 * n + 2];
        }
    }
    caller[t] = (int32_t)n;
    cx_s[t] = cx;
    cy_s[t] = cy;
    cz_s[t] = cz;

    unsigned long long mask = 0;
    unsigned long long cnt = 0;
    for (int k = 0; k < K; ++k) {
        int32_t v = N32;
        if (n >= 0) v = probe(a, n, cx, cy, cz, k);
        if (v != N32) {
            ++cnt;
            if (k < 63) mask |= 1ull << k;
        }
        if (K <= kLdsK) nbs[k][t] = v;
    }
    keys[t] = (n < 0) ? ~0ull : mask;
    // valid-pair count of the tile
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) cnt_s[wv] = cnt;
    __syncthreads();
    if (t == 0) {
        unsigned long long c = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
        if (c) atomicAdd(&a.info->valid_pairs, c);
    }
    // stable rank of this row's key inside the tile
    const unsigned long long my = keys[t];
    int rank = 0;
    for (int u = 0; u < kTileRows; ++u) {
        const unsigned long long o = keys[u];
        rank += (o < my) || (o == my && u < t);
    }
    rowsrc[rank] = t;
    __syncthreads();

    const int src = rowsrc[t];               // this thread now writes sorted row t
    const int64_t out_row = tile * kTileRows + t;
    const int32_t src_n = caller[src];
    a.order[out_row] = src_n;
    for (int k = 0; k < K; ++k) {
        int32_t v;
        if (K <= kLdsK) {
            v = nbs[k][src];
        } else {
            v = (src_n >= 0) ? probe(a, src_n, cx_s[src], cy_s[src], cz_s[src], k) : N32;
        }
        a.nbr_m[(int64_t)k * a.Npad + out_row] = v;
        const uint64_t bal = __ballot(v != N32);
        if (lane == 0) {
            uint8_t b = 0;
            for (int q = 0; q < 4; ++q) b |= (uint8_t)(((bal >> (16 * q)) & 0xffffull) != 0) << q;
            wbits[k & 255][wv] = b;
        }
        if ((k & 255) == 255 || k == K - 1) {
            __syncthreads();
            const int kb = k & ~255;
            if (t <= (k - kb)) {
                const int kk = kb + t;
                uint16_t m16 = (uint16_t)(wbits[t][0] | (wbits[t][1] << 4) | (wbits[t][2] << 8) |
                                          (wbits[t][3] << 12));
                a.blkmask[tile * K + kk] = m16;
            }
            __syncthreads();
        }
    }
}

__global__ void k_export(const int32_t* __restrict__ nbr_m, const int32_t* __restrict__ order,
                         int64_t N, int64_t Npad, int32_t* __restrict__ nbr_out,
                         int32_t* __restrict__ order_out) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int k = blockIdx.y;
    if (j >= N) return;  // padding rows are all at the end of the schedule
    const int32_t n = order[j];
    if ((uint32_t)n >= (uint32_t)N) return;
    if (nbr_out) nbr_out[(int64_t)k * N + n] = nbr_m[(int64_t)k * Npad + j];
    if (order_out && k == 0) order_out[j] = n;
}

inline int ceil_log2(uint64_t v) {
    int l = 0;
    while ((1ull << l) < v) ++l;
    return l;
}

inline hipError_t fill_u32(void* p, int64_t n, uint32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    k_fill_u32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((uint32_t*)p, n, v);
    return hipGetLastError();
}

hipError_t run_tile_query(QueryArgs qa, const ArenaLayout& al, hipStream_t stream) {
    k_tile_query<<<dim3((unsigned)al.ntiles), dim3(kTileRows), 0, stream>>>(qa);
    return hipGetLastError();
}

}  // namespace

int cube_side(int K) {
    if (K < 1) return -1;
    for (int s = 1; (int64_t)s * s * s <= K; s += 2)
        if (s * s * s == K) return s;
    return -1;
}

ArenaLayout arena_layout(int64_t N, int K) {
    ArenaLayout l;
    l.Npad = round_up(N > 0 ? N : 1, kTileRows);
    l.ntiles = l.Npad / kTileRows;
    size_t off = 0;
    l.nbr_off = off;
    off = align_up(off + (size_t)4 * K * l.Npad, 256);
    l.order_off = off;
    off = align_up(off + (size_t)4 * l.Npad, 256);
    l.mask_off = off;
    off = align_up(off + (size_t)2 * K * l.ntiles, 256);
    l.info_off = off;
    off = align_up(off + sizeof(MapInfo), 256);
    l.total = off;
    return l;
}

WorkspaceLayout workspace_layout(int64_t N) {
    WorkspaceLayout l;
    const int64_t n = N > 0 ? N : 1;
    l.nsort_blocks = (n + kSortChunk - 1) / kSortChunk;
    l.log2_cap = ceil_log2((uint64_t)(2 * n));
    if (l.log2_cap < 10) l.log2_cap = 10;
    size_t off = 0;
    l.codes0 = off;
    off = align_up(off + 8 * (size_t)n, 256);
    l.codes1 = off;
    off = align_up(off + 8 * (size_t)n, 256);
    l.idx0 = off;
    off = align_up(off + 4 * (size_t)n, 256);
    l.idx1 = off;
    off = align_up(off + 4 * (size_t)n, 256);
    l.hist = off;
    off = align_up(off + 4 * (size_t)kRadix * l.nsort_blocks, 256);
    l.totals = off;
    off = align_up(off + 4 * (size_t)kRadix, 256);
    l.table = off;
    off = align_up(off + sizeof(HashSlot) * ((size_t)1 << l.log2_cap), 256);
    l.flags = off;
    off = align_up(off + sizeof(BuildFlags), 256);
    l.total = off;
    return l;
}

#define SPC_TRY(x)                         \
    do {                                   \
        hipError_t e_ = (x);               \
        if (e_ != hipSuccess) return e_;   \
    } while (0)

hipError_t launch_build(const int32_t* coords, int64_t N, int K, int dilation, int side,
                        const ArenaLayout& al, char* arena, const WorkspaceLayout& wl, char* ws,
                        hipStream_t stream, BuildFlags* host_flags) {
    uint64_t* codes[2] = {(uint64_t*)(ws + wl.codes0), (uint64_t*)(ws + wl.codes1)};
    uint32_t* idx[2] = {(uint32_t*)(ws + wl.idx0), (uint32_t*)(ws + wl.idx1)};
    uint32_t* hist = (uint32_t*)(ws + wl.hist);
    uint32_t* totals = (uint32_t*)(ws + wl.totals);
    HashSlot* table = (HashSlot*)(ws + wl.table);
    BuildFlags* flags = (BuildFlags*)(ws + wl.flags);
    MapInfo* info = (MapInfo*)(arena + al.info_off);

    SPC_TRY(fill_u32(table, (int64_t)4 << wl.log2_cap, 0xffffffffu, stream));
    SPC_TRY(fill_u32(flags, sizeof(BuildFlags) / 4, 0u, stream));
    SPC_TRY(fill_u32(info, sizeof(MapInfo) / 4, 0u, stream));

    const unsigned pblocks = (unsigned)((N + 255) / 256);
    k_pack_insert<<<dim3(pblocks), dim3(256), 0, stream>>>(coords, N, codes[0], idx[0], table,
                                                            wl.log2_cap, flags);
    SPC_TRY(hipGetLastError());
    SPC_TRY(hipMemcpyAsync(host_flags, flags, sizeof(BuildFlags), hipMemcpyDeviceToHost, stream));
    SPC_TRY(hipStreamSynchronize(stream));
    if (host_flags->range_error || host_flags->duplicate) return hipSuccess;

    // sort on the bits that differ across the set; higher bits are common
    const uint64_t x = host_flags->morton_xor_or;
    int bits = 0;
    while (bits < 64 && (x >> bits)) ++bits;
    const int passes = (bits + kRadixBits - 1) / kRadixBits;
    int cur = 0;
    for (int p = 0; p < passes; ++p) {
        const int shift = p * kRadixBits;
        k_radix_hist<<<dim3((unsigned)wl.nsort_blocks), dim3(kSortThreads), 0, stream>>>(
            codes[cur], N, shift, hist, wl.nsort_blocks);
        SPC_TRY(hipGetLastError());
        k_radix_rowscan<<<dim3(kRadix), dim3(256), 0, stream>>>(hist, wl.nsort_blocks, totals);
        SPC_TRY(hipGetLastError());
        k_radix_scatter<<<dim3((unsigned)wl.nsort_blocks), dim3(kSortThreads), 0, stream>>>(
            codes[cur], idx[cur], N, shift, hist, wl.nsort_blocks, totals, codes[cur ^ 1],
            idx[cur ^ 1]);
        SPC_TRY(hipGetLastError());
        cur ^= 1;
    }

    QueryArgs qa;
    qa.coords = coords;
    qa.morton_idx = idx[cur];
    qa.table = table;
    qa.nbr_in = nullptr;
    qa.N = N;
    qa.Npad = al.Npad;
    qa.K = K;
    qa.side = side;
    qa.dilation = dilation;
    qa.log2_cap = wl.log2_cap;
    qa.mode = 0;
    qa.nbr_m = (int32_t*)(arena + al.nbr_off);
    qa.order = (int32_t*)(arena + al.order_off);
    qa.blkmask = (uint16_t*)(arena + al.mask_off);
    qa.info = info;
    return run_tile_query(qa, al, stream);
}

hipError_t launch_wrap(const int32_t* nbr, int64_t N, int K, const ArenaLayout& al, char* arena,
                       hipStream_t stream) {
    MapInfo* info = (MapInfo*)(arena + al.info_off);
    SPC_TRY(fill_u32(info, sizeof(MapInfo) / 4, 0u, stream));
    QueryArgs qa;
    qa.coords = nullptr;
    qa.morton_idx = nullptr;
    qa.table = nullptr;
    qa.nbr_in = nbr;
    qa.N = N;
    qa.Npad = al.Npad;
    qa.K = K;
    qa.side = 1;
    qa.dilation = 1;
    qa.log2_cap = 10;
    qa.mode = 1;
    qa.nbr_m = (int32_t*)(arena + al.nbr_off);
    qa.order = (int32_t*)(arena + al.order_off);
    qa.blkmask = (uint16_t*)(arena + al.mask_off);
    qa.info = info;
    return run_tile_query(qa, al, stream);
}

hipError_t launch_export(const int32_t* nbr_m, const int32_t* order, int64_t N, int64_t Npad, int K,
                         int32_t* nbr_out, int32_t* order_out, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)(nbr_out ? K : 1));
    k_export<<<grid, dim3(256), 0, stream>>>(nbr_m, order, N, Npad, nbr_out, order_out);
    return hipGetLastError();
}

}  // namespace spc
