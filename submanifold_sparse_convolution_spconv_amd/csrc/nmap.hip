// Neighbour-map builder for gfx950.
//
// The page ("mlx_backend/sparse_conv_metal.py", `sparse_conv_metal` wrapper
// docstring) takes the (K, N) int32 map, sentinel N, as an input and does not
// show how it is made.  This builder produces it on the GPU:
//
//   1. pack:   range-check each coordinate and compute its 63-bit Morton code;
//              OR together (code ^ code of voxel 0) to find the varying bits.
//   2. sort:   LSD radix sort of (Morton code, caller index) on those bits
//              (8 bits per pass) -> voxels in Morton order.
//   3. bricks: the voxels of one 4x4x4 brick are consecutive in that order
//              (the low 6 Morton bits are the cell inside the brick).  One
//              thread per brick inserts (brick code -> first position, 64-bit
//              cell mask) into an open-addressing hash table (64-bit
//              compare-and-swap, linear probing, load <= 1/2), sized on the
//              device from the brick count; equal adjacent codes flag a
//              duplicate coordinate.  On surfaces a brick holds ~16 voxels, so
//              the table is small enough to stay in L2.
//   4. query:  one workgroup per 256-row tile of the Morton order looks up the
//              K neighbours of each row: a neighbour is present iff its cell
//              bit is set in its brick's mask, and its Morton position is the
//              brick start plus the set bits below its cell.  For the 3x3x3
//              stencil at dilation <= 2 a row's neighbours lie in at most 8
//              bricks, which are probed together.  The tile's rows are then
//              sorted by their
//              K-bit validity mask (rows with equal patterns end up in the same
//              16-row blocks, so more blocks are entirely missing for a given
//              offset and the forward can skip them), then writes the map in
//              that row order plus one 16-bit block mask per (tile, k).
//
// All writes are plain vector stores and vector atomics.
#include "spconv_internal.h"

namespace spc {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Inverse of spread3: gather bits 0, 3, 6, ... of x into the low 21 bits.
__device__ __forceinline__ uint32_t compact3(uint64_t x) {
    x &= 0x1249249249249249ull;
    x = (x ^ (x >> 2)) & 0x10c30c30c30c30c3ull;
    x = (x ^ (x >> 4)) & 0x100f00f00f00f00full;
    x = (x ^ (x >> 8)) & 0x001f0000ff0000ffull;
    x = (x ^ (x >> 16)) & 0x001f00000000ffffull;
    x = (x ^ (x >> 32)) & 0x00000000001fffffull;
    return (uint32_t)x;
}

// Sort (key, idx) pairs ascending (key first, then idx) across the 64 lanes
// of a wave: a bitonic network, partners exchanged with cross-lane shuffles.
// idx values are distinct, so the order is total.
__device__ __forceinline__ void wave_sort64(unsigned long long& key, uint32_t& idx, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t olo = (uint32_t)__shfl_xor((int)(uint32_t)key, j);
            const uint32_t ohi = (uint32_t)__shfl_xor((int)(uint32_t)(key >> 32), j);
            const uint32_t oi = (uint32_t)__shfl_xor((int)idx, j);
            const unsigned long long ok = ((unsigned long long)ohi << 32) | olo;
            const bool less = ok < key || (ok == key && oi < idx);     // partner before me
            const bool ascending = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            if ((lower == ascending) ? less : !less) {
                key = ok;
                idx = oi;
            }
        }
    }
}

// Brick of biased coordinates (u >> 2 per axis) -> its Morton code, equal to
// the voxel Morton code >> 6.
__device__ __forceinline__ uint64_t brick_key(uint32_t bx, uint32_t by, uint32_t bz) {
    return spread3(bz) | (spread3(by) << 1) | (spread3(bx) << 2);
}

// Cell of biased coordinates inside their brick: the low 6 Morton bits.
__device__ __forceinline__ uint32_t cell_of(uint32_t ux, uint32_t uy, uint32_t uz) {
    return (uz & 1u) | ((uy & 1u) << 1) | ((ux & 1u) << 2) | ((uz & 2u) << 2) | ((uy & 2u) << 3) |
           ((ux & 2u) << 4);
}

__device__ __forceinline__ uint32_t brick_home(unsigned long long key, int log2_cap) {
    return (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> (64 - log2_cap));
}

__device__ __forceinline__ int ceil_log2_dev(uint32_t v) {
    return v <= 1 ? 0 : 32 - __clz(v - 1);
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

// Grid-stride over voxels; one atomic per block for the OR of code
// differences (same-address atomics from every wave would serialise).
__global__ void __launch_bounds__(256) k_pack(const int32_t* __restrict__ coords, int64_t N,
                                              uint64_t* __restrict__ codes,
                                              uint32_t* __restrict__ idx, BuildFlags* flags) {
    __shared__ uint64_t part[4];
    const uint64_t code0 = morton3(coords[0], coords[1], coords[2]);
    uint64_t diff = 0;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int x = coords[3 * i], y = coords[3 * i + 1], z = coords[3 * i + 2];
        idx[i] = (uint32_t)i;
        if (!coord_ok(x) || !coord_ok(y) || !coord_ok(z)) {
            bad = true;
            codes[i] = 0;
        } else {
            const uint64_t code = morton3(x, y, z);
            codes[i] = code;
            diff |= code ^ code0;
        }
    }
    if (bad) atomicOr(&flags->range_error, 1u);
    diff = wave_or(diff);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = diff;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t d = part[0] | part[1] | part[2] | part[3];
        if (d) atomicOr((unsigned long long*)&flags->morton_xor_or, (unsigned long long)d);
    }
}

// Brick heads in the sorted codes: count them, flag equal neighbours.
__global__ void __launch_bounds__(256) k_brick_count(const uint64_t* __restrict__ codes, int64_t N,
                                                     BuildFlags* flags) {
    __shared__ uint32_t part[4];
    uint32_t heads = 0;
    bool dup = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t c = codes[i];
        if (i == 0) {
            ++heads;
        } else {
            const uint64_t p = codes[i - 1];
            heads += (c >> 6) != (p >> 6);
            dup |= c == p;
        }
    }
    if (dup) atomicOr(&flags->duplicate, 1u);
    for (int o = 32; o > 0; o >>= 1) heads += __shfl_xor(heads, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = heads;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t h = part[0] + part[1] + part[2] + part[3];
        if (h) atomicAdd(&flags->nbricks, h);
    }
}

// Size the brick table from the count (load <= 1/2, at least 2^10 slots, at
// most the workspace's 2^max_log2) and mark its slots empty.
__global__ void __launch_bounds__(256) k_brick_fill(BrickSlot* table, int max_log2, BuildFlags* flags) {
    int L = ceil_log2_dev(2u * flags->nbricks);
    L = L < 10 ? 10 : (L > max_log2 ? max_log2 : L);
    if (blockIdx.x == 0 && threadIdx.x == 0) flags->log2_bricks = (uint32_t)L;
    const int64_t cap = (int64_t)1 << L;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cap;
         i += (int64_t)gridDim.x * blockDim.x)
        table[i].key = kEmptyKey;
}

// One thread per brick head: OR the cells of its run, insert the brick.
__global__ void __launch_bounds__(256) k_brick_insert(const uint64_t* __restrict__ codes, int64_t N,
                                                      BrickSlot* table, const BuildFlags* flags) {
    const int L = (int)flags->log2_bricks;
    const uint32_t cap_mask = (1u << L) - 1u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t key = codes[i] >> 6;
        if (i > 0 && (codes[i - 1] >> 6) == key) continue;
        unsigned long long mask = 0;
        for (int64_t j = i; j < N && (codes[j] >> 6) == key; ++j) mask |= 1ull << (codes[j] & 63u);
        uint32_t s = brick_home(key, L);
        for (;;) {  // terminates: load <= 1/2 leaves empty slots and the probe is linear
            const unsigned long long prev = atomicCAS(&table[s].key, kEmptyKey, (unsigned long long)key);
            if (prev == kEmptyKey || prev == key) {
                table[s].start = (uint32_t)i;
                table[s].mask = mask;
                break;
            }
            s = (s + 1) & cap_mask;
        }
    }
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
    const uint64_t* codes;        // mode 0: sorted Morton codes (coordinates are decoded from them)
    const uint32_t* morton_idx;   // mode 0: Morton position -> caller index
    const BrickSlot* table;       // mode 0
    const BuildFlags* bflags;     // mode 0: capacity of the brick table in use
    const int32_t* nbr_in;        // mode 1, (K, N)
    int64_t N, Npad;
    int K, side, dilation, mode;
    int32_t* nbr_m;
    int32_t* order;
    uint16_t* blkmask;
    MapInfo* info;
};

constexpr int kProbeChunk = 9;

// Look up M bricks at once: the first slot of every wanted key is loaded
// before any is examined; collisions then walk on (linear probing).
// mask = 0 for a brick that is not in the table.
template <int M>
__device__ __forceinline__ void find_bricks(const BrickSlot* table, int L,
                                            const unsigned long long (&key)[M], const bool (&want)[M],
                                            uint32_t (&start)[M], unsigned long long (&mask)[M]) {
    const uint32_t cap_mask = (1u << L) - 1u;
    uint32_t slot[M];
    u32x4 lo[M], hi[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        start[i] = 0;
        mask[i] = 0;
        if (want[i]) {
            slot[i] = brick_home(key[i], L);
            lo[i] = *(const u32x4*)&table[slot[i]];
            hi[i] = *((const u32x4*)&table[slot[i]] + 1);
        }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
        if (!want[i]) continue;
        for (;;) {  // terminates: load <= 1/2 leaves empty slots and the probe is linear
            const unsigned long long kk = ((unsigned long long)lo[i][1] << 32) | lo[i][0];
            if (kk == key[i]) {
                start[i] = lo[i][2];
                mask[i] = ((unsigned long long)hi[i][1] << 32) | hi[i][0];
                break;
            }
            if (kk == kEmptyKey) break;
            slot[i] = (slot[i] + 1) & cap_mask;
            lo[i] = *(const u32x4*)&table[slot[i]];
            hi[i] = *((const u32x4*)&table[slot[i]] + 1);
        }
    }
}

// Caller index of the voxel in cell `cell` of a brick (start, mask), or N.
__device__ __forceinline__ int32_t cell_voxel(const QueryArgs& a, bool ok, uint32_t start,
                                              unsigned long long mask, uint32_t cell) {
    if (!ok || !((mask >> cell) & 1ull)) return (int32_t)a.N;
    return (int32_t)a.morton_idx[start + __popcll(mask & ((1ull << cell) - 1ull))];
}

// 3x3x3 stencil at dilation <= 2: along each axis the three offsets fall in at
// most two bricks (c0 below, c1 above), so a row's 27 neighbours lie in the 8
// bricks (c0|c1)^3, which are looked up together.
__device__ __forceinline__ void neighbours27(const QueryArgs& a, int L, int cx, int cy, int cz,
                                             int32_t (&v)[27]) {
    const uint32_t d = (uint32_t)a.dilation;
    const uint32_t top = 2u * (uint32_t)kCoordBias;
    const uint32_t u[3] = {(uint32_t)(cx + kCoordBias), (uint32_t)(cy + kCoordBias), (uint32_t)(cz + kCoordBias)};
    bool lo_ok[3], hi_ok[3];
    uint32_t c0[3], c1[3];
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
        lo_ok[ax] = u[ax] >= d;
        hi_ok[ax] = u[ax] + d < top;
        c0[ax] = (lo_ok[ax] ? u[ax] - d : u[ax]) >> 2;
        c1[ax] = (hi_ok[ax] ? u[ax] + d : u[ax]) >> 2;
    }
    unsigned long long key[8];
    bool want[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        key[i] = brick_key((i & 4) ? c1[0] : c0[0], (i & 2) ? c1[1] : c0[1], (i & 1) ? c1[2] : c0[2]);
        want[i] = true;
    }
    uint32_t st[8];
    unsigned long long mk[8];
    find_bricks<8>(a.table, L, key, want, st, mk);
#pragma unroll
    for (int k = 0; k < 27; ++k) {
        const int o[3] = {k / 9 - 1, (k / 3) % 3 - 1, k % 3 - 1};
        bool ok = true;
        uint32_t nn[3];
        int combo = 0;
#pragma unroll
        for (int ax = 0; ax < 3; ++ax) {
            if (o[ax] < 0) {
                ok = ok && lo_ok[ax];
                nn[ax] = u[ax] - d;
            } else if (o[ax] > 0) {
                ok = ok && hi_ok[ax];
                nn[ax] = u[ax] + d;
            } else {
                nn[ax] = u[ax];
            }
            combo |= ((nn[ax] >> 2) != c0[ax] ? 1 : 0) << (2 - ax);
        }
        uint32_t bs = 0;
        unsigned long long bm = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (combo == i) {
                bs = st[i];
                bm = mk[i];
            }
        v[k] = cell_voxel(a, ok, bs, bm, cell_of(nn[0], nn[1], nn[2]));
    }
}

// Any odd-cube stencil and dilation: offsets k0 .. k0+nk-1 (nk <= kProbeChunk),
// one brick lookup per offset, all in flight together.  Mode 1 reads the
// caller's map instead.
__device__ __forceinline__ void neighbours_chunk(const QueryArgs& a, int L, int64_t n, int cx, int cy,
                                                 int cz, int k0, int nk, int32_t (&v)[kProbeChunk]) {
    const int N32 = (int)a.N;
    if (a.mode == 1) {
#pragma unroll
        for (int i = 0; i < kProbeChunk; ++i) {
            if (i < nk) {
                const int32_t r = a.nbr_in[(int64_t)(k0 + i) * a.N + n];
                v[i] = ((uint32_t)r < (uint32_t)N32) ? r : N32;
            }
        }
        return;
    }
    const int s = a.side, rr = (a.side - 1) >> 1;
    unsigned long long key[kProbeChunk];
    bool want[kProbeChunk];
    uint32_t cell[kProbeChunk];
#pragma unroll
    for (int i = 0; i < kProbeChunk; ++i) {
        want[i] = false;
        key[i] = 0;
        cell[i] = 0;
        if (i < nk) {
            const int k = k0 + i;
            const int dc = k % s, db = (k / s) % s, da = k / (s * s);
            const int x = cx + a.dilation * (da - rr);
            const int y = cy + a.dilation * (db - rr);
            const int z = cz + a.dilation * (dc - rr);
            if (coord_ok(x) && coord_ok(y) && coord_ok(z)) {
                const uint32_t ux = (uint32_t)(x + kCoordBias), uy = (uint32_t)(y + kCoordBias),
                               uz = (uint32_t)(z + kCoordBias);
                want[i] = true;
                key[i] = brick_key(ux >> 2, uy >> 2, uz >> 2);
                cell[i] = cell_of(ux, uy, uz);
            }
        }
    }
    uint32_t st[kProbeChunk];
    unsigned long long mk[kProbeChunk];
    find_bricks<kProbeChunk>(a.table, L, key, want, st, mk);
#pragma unroll
    for (int i = 0; i < kProbeChunk; ++i)
        if (i < nk) v[i] = cell_voxel(a, want[i], st[i], mk[i], cell[i]);
}

__global__ void __launch_bounds__(kTileRows) k_tile_query(QueryArgs a) {
    __shared__ int32_t nbs[kLdsK][kTileRows];
    __shared__ unsigned long long keys[kTileRows];
    __shared__ int32_t rowsrc[kTileRows];     // sorted position -> original thread
    __shared__ int32_t caller[kTileRows];     // original thread -> caller index (-1 pad)
    __shared__ int cx_s[kTileRows], cy_s[kTileRows], cz_s[kTileRows];
    __shared__ uint8_t wbits[256][4];
    __shared__ unsigned long long cnt_s[4];
    __shared__ unsigned long long run_k[kTileRows];   // per-wave sorted runs of (key, row)
    __shared__ uint32_t run_i[kTileRows];

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
            // the sorted Morton code carries the coordinates (biased by 2^20)
            const uint64_t code = a.codes[j];
            cx = (int)compact3(code >> 2) - kCoordBias;
            cy = (int)compact3(code >> 1) - kCoordBias;
            cz = (int)compact3(code) - kCoordBias;
        }
    }
    caller[t] = (int32_t)n;
    cx_s[t] = cx;
    cy_s[t] = cy;
    cz_s[t] = cz;

    const int L = a.mode == 0 ? (int)a.bflags->log2_bricks : 0;
    unsigned long long mask = 0;
    unsigned long long cnt = 0;
    if (a.mode == 0 && a.side == 3 && a.dilation <= 2) {
        int32_t v[27];
        if (n >= 0) {
            neighbours27(a, L, cx, cy, cz, v);
        } else {
#pragma unroll
            for (int k = 0; k < 27; ++k) v[k] = N32;
        }
#pragma unroll
        for (int k = 0; k < 27; ++k) {
            if (v[k] != N32) {
                ++cnt;
                mask |= 1ull << k;
            }
            nbs[k][t] = v[k];
        }
    } else {
        for (int k0 = 0; k0 < K; k0 += kProbeChunk) {
            const int nk = K - k0 < kProbeChunk ? K - k0 : kProbeChunk;
            int32_t v[kProbeChunk];
            if (n >= 0) {
                neighbours_chunk(a, L, n, cx, cy, cz, k0, nk, v);
            } else {
#pragma unroll
                for (int i = 0; i < kProbeChunk; ++i) v[i] = N32;
            }
#pragma unroll
            for (int i = 0; i < kProbeChunk; ++i) {
                if (i < nk) {
                    const int k = k0 + i;
                    if (v[i] != N32) {
                        ++cnt;
                        if (k < 63) mask |= 1ull << k;
                    }
                    if (K <= kLdsK) nbs[k][t] = v[i];
                }
            }
        }
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
    // stable rank of this row's key inside the tile: each wave sorts its 64
    // (key, row) pairs, and a row's rank is the number of pairs before it in
    // the four sorted runs (binary searches)
    const unsigned long long my = keys[t];
    {
        unsigned long long sk = my;
        uint32_t si = (uint32_t)t;
        wave_sort64(sk, si, lane);
        run_k[t] = sk;
        run_i[t] = si;
    }
    __syncthreads();
    int rank = 0;
#pragma unroll
    for (int w2 = 0; w2 < kTileRows / 64; ++w2) {
        const int b0 = w2 * 64;
        int lo = 0;
#pragma unroll
        for (int step = 32; step > 0; step >>= 1) {
            const int q = b0 + lo + step - 1;
            const unsigned long long o = run_k[q];
            if (o < my || (o == my && run_i[q] < (uint32_t)t)) lo += step;
        }
        const unsigned long long o = run_k[b0 + lo];
        if (lo < 64 && (o < my || (o == my && run_i[b0 + lo] < (uint32_t)t))) ++lo;
        rank += lo;
    }
    rowsrc[rank] = t;
    __syncthreads();

    const int src = rowsrc[t];               // this thread now writes sorted row t
    const int64_t out_row = tile * kTileRows + t;
    const int32_t src_n = caller[src];
    a.order[out_row] = src_n;
    int32_t vchunk[kProbeChunk];
    for (int k = 0; k < K; ++k) {
        int32_t v;
        if (K <= kLdsK) {
            v = nbs[k][src];
        } else {
            // more offsets than LDS holds: probe again, a chunk at a time
            const int i = k % kProbeChunk;
            if (i == 0) {
                const int nk = K - k < kProbeChunk ? K - k : kProbeChunk;
                if (src_n >= 0) {
                    neighbours_chunk(a, L, src_n, cx_s[src], cy_s[src], cz_s[src], k, nk, vchunk);
                } else {
#pragma unroll
                    for (int j = 0; j < kProbeChunk; ++j) vchunk[j] = N32;
                }
            }
            int32_t sel = N32;
#pragma unroll
            for (int j = 0; j < kProbeChunk; ++j)
                if (j == i) sel = vchunk[j];
            v = sel;
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
    // brick table: at most N bricks, load <= 1/2; only the part the actual
    // brick count needs is cleared and probed
    off = align_up(off + sizeof(BrickSlot) * ((size_t)1 << l.log2_cap), 256);
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
                        hipStream_t stream, BuildFlags* host_flags,
                        unsigned long long* host_valid_pairs) {
    uint64_t* codes[2] = {(uint64_t*)(ws + wl.codes0), (uint64_t*)(ws + wl.codes1)};
    uint32_t* idx[2] = {(uint32_t*)(ws + wl.idx0), (uint32_t*)(ws + wl.idx1)};
    uint32_t* hist = (uint32_t*)(ws + wl.hist);
    uint32_t* totals = (uint32_t*)(ws + wl.totals);
    BrickSlot* table = (BrickSlot*)(ws + wl.table);
    BuildFlags* flags = (BuildFlags*)(ws + wl.flags);
    MapInfo* info = (MapInfo*)(arena + al.info_off);

    SPC_TRY(fill_u32(flags, sizeof(BuildFlags) / 4, 0u, stream));
    SPC_TRY(fill_u32(info, sizeof(MapInfo) / 4, 0u, stream));

    const unsigned pblocks = (unsigned)((N + 255) / 256);
    k_pack<<<dim3(pblocks < 1024 ? pblocks : 1024), dim3(256), 0, stream>>>(coords, N, codes[0], idx[0],
                                                                             flags);
    SPC_TRY(hipGetLastError());
    SPC_TRY(hipMemcpyAsync(host_flags, flags, sizeof(BuildFlags), hipMemcpyDeviceToHost, stream));
    SPC_TRY(hipStreamSynchronize(stream));
    if (host_flags->range_error) return hipSuccess;

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

    const unsigned gblocks = pblocks < 2048 ? pblocks : 2048;
    k_brick_count<<<dim3(gblocks), dim3(256), 0, stream>>>(codes[cur], N, flags);
    SPC_TRY(hipGetLastError());
    k_brick_fill<<<dim3(gblocks), dim3(256), 0, stream>>>(table, wl.log2_cap, flags);
    SPC_TRY(hipGetLastError());
    k_brick_insert<<<dim3(gblocks), dim3(256), 0, stream>>>(codes[cur], N, table, flags);
    SPC_TRY(hipGetLastError());

    QueryArgs qa;
    qa.coords = coords;
    qa.codes = codes[cur];
    qa.morton_idx = idx[cur];
    qa.table = table;
    qa.bflags = flags;
    qa.nbr_in = nullptr;
    qa.N = N;
    qa.Npad = al.Npad;
    qa.K = K;
    qa.side = side;
    qa.dilation = dilation;
    qa.mode = 0;
    qa.nbr_m = (int32_t*)(arena + al.nbr_off);
    qa.order = (int32_t*)(arena + al.order_off);
    qa.blkmask = (uint16_t*)(arena + al.mask_off);
    qa.info = info;
    SPC_TRY(run_tile_query(qa, al, stream));
    // second round trip: duplicate flag and the valid-pair count
    SPC_TRY(hipMemcpyAsync(host_flags, flags, sizeof(BuildFlags), hipMemcpyDeviceToHost, stream));
    SPC_TRY(hipMemcpyAsync(host_valid_pairs, &info->valid_pairs, sizeof(unsigned long long),
                           hipMemcpyDeviceToHost, stream));
    return hipStreamSynchronize(stream);
}

hipError_t launch_wrap(const int32_t* nbr, int64_t N, int K, const ArenaLayout& al, char* arena,
                       hipStream_t stream) {
    MapInfo* info = (MapInfo*)(arena + al.info_off);
    SPC_TRY(fill_u32(info, sizeof(MapInfo) / 4, 0u, stream));
    QueryArgs qa;
    qa.coords = nullptr;
    qa.codes = nullptr;
    qa.morton_idx = nullptr;
    qa.table = nullptr;
    qa.bflags = nullptr;
    qa.nbr_in = nbr;
    qa.N = N;
    qa.Npad = al.Npad;
    qa.K = K;
    qa.side = 1;
    qa.dilation = 1;
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
