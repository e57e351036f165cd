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
//              bricks, which are probed together.  The rows of each half
//              tile (128 rows) are then sorted by their K-bit validity mask
//              (rows with equal patterns end up in the same 16-row blocks, so
//              more blocks are entirely missing for a given offset and the
//              forward can skip them), then the map is written in that row
//              order plus one 16-bit block mask per (tile, k).
//   5. lists:  per half tile, the distinct rows its rows have as present
//              neighbours and each (row, offset)'s slot among them, which the
//              forward stages in LDS once per half tile.
//
// All writes are plain vector stores and vector atomics.
#include <algorithm>

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

// Coordinates as the caller gives them: (N, 3) x, y, z, or (N, 4) b, x, y, z
// for B batches.  Batch b occupies its own slab of S = 2^log2S x-values of
// the [-2^20, 2^20) range: x' = x + b*S - 2^20 + S/2, with x in
// [-S/2 + margin, S/2 - margin), margin = the stencil's reach, so no stencil
// reaches from one batch's slab into another's.
struct CoordForm {
    int stride;     // 3 or 4
    int B;          // batches (stride 4)
    int log2S;      // slab width (stride 4)
    int margin;     // dilation * stencil radius (stride 4)
};

__device__ __forceinline__ bool fetch_coord(const int32_t* __restrict__ coords, const CoordForm& f, int64_t i,
                                            int& x, int& y, int& z) {
    if (f.stride == 3) {
        x = coords[3 * i];
        y = coords[3 * i + 1];
        z = coords[3 * i + 2];
        return coord_ok(x) && coord_ok(y) && coord_ok(z);
    }
    const int b = coords[4 * i];
    const int xb = coords[4 * i + 1];
    y = coords[4 * i + 2];
    z = coords[4 * i + 3];
    const int half = 1 << (f.log2S - 1);
    const bool ok = b >= 0 && b < f.B && xb >= -half + f.margin && xb < half - f.margin && coord_ok(y) && coord_ok(z);
    x = ok ? xb + (int)(((uint32_t)b << f.log2S) - (uint32_t)kCoordBias + (uint32_t)half) : 0;
    return ok;
}

// One workgroup per sort block of kSortChunk voxels (the chunk the first radix
// pass reads): Morton codes, caller indices, the block's histogram of the
// first digit, and a per-block partial of the OR of code differences and of
// the range check (reduced by the first pass's scan kernel).
__global__ void __launch_bounds__(kSortThreads) k_pack(const int32_t* __restrict__ coords, CoordForm form, int64_t N,
                                                       uint64_t* __restrict__ codes,
                                                       uint32_t* __restrict__ idx,
                                                       uint32_t* __restrict__ hist, int64_t nblk,
                                                       PackPart* __restrict__ part) {
    constexpr int NW = kSortThreads / 64;
    __shared__ uint32_t h[kRadix];
    __shared__ uint64_t wor[NW];
    __shared__ uint32_t wbad[NW];
    const int t = threadIdx.x;
    if (t < kRadix) h[t] = 0;
    int x0, y0, z0;
    fetch_coord(coords, form, 0, x0, y0, z0);
    const uint64_t code0 = morton3(x0, y0, z0);
    const int64_t b0 = (int64_t)blockIdx.x * kSortChunk;
    uint64_t c[kSortItems];
    uint64_t diff = 0;
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t i = b0 + (int64_t)r * kSortThreads + t;
        c[r] = 0;
        if (i < N) {
            int x, y, z;
            if (!fetch_coord(coords, form, i, x, y, z)) {
                bad = true;
            } else {
                c[r] = morton3(x, y, z);
                diff |= c[r] ^ code0;
            }
            codes[i] = c[r];
            idx[i] = (uint32_t)i;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t i = b0 + (int64_t)r * kSortThreads + t;
        if (i < N) atomicAdd(&h[(uint32_t)c[r] & (kRadix - 1)], 1u);
    }
    diff = wave_or(diff);
    const uint64_t anybad = __ballot(bad);
    if ((t & 63) == 0) {
        wor[t >> 6] = diff;
        wbad[t >> 6] = anybad != 0;
    }
    __syncthreads();
    if (t < kRadix) hist[(int64_t)t * nblk + blockIdx.x] = h[t];
    if (t == 0) {
        PackPart pp;
        pp.xor_or = 0;
        pp.bad = 0;
        for (int w = 0; w < NW; ++w) {
            pp.xor_or |= wor[w];
            pp.bad |= wbad[w];
        }
        pp.pad = 0;
        part[blockIdx.x] = pp;
    }
}

// Brick heads in the sorted codes: per-workgroup count, and a flag for equal
// neighbours (a duplicate coordinate).  kCountBlocks workgroups, grid-stride.
__global__ void __launch_bounds__(256) k_brick_count(const uint64_t* __restrict__ codes, int64_t N,
                                                     CountPart* __restrict__ part) {
    __shared__ uint32_t wh[4], wd[4];
    uint32_t heads = 0;
    bool dup = false;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < N; i0 += 4 * stride) {
        uint64_t c[4], p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // four independent loads in flight
            const int64_t i = i0 + u * stride;
            c[u] = i < N ? codes[i] : 0;
            p[u] = (i > 0 && i < N) ? codes[i - 1] : ~0ull;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * stride;
            if (i < N) {
                heads += (i == 0) || (c[u] >> 6) != (p[u] >> 6);
                dup |= i > 0 && c[u] == p[u];
            }
        }
    }
    for (int o = 32; o > 0; o >>= 1) heads += __shfl_xor(heads, o);
    const uint64_t anydup = __ballot(dup);
    if ((threadIdx.x & 63) == 0) {
        wh[threadIdx.x >> 6] = heads;
        wd[threadIdx.x >> 6] = anydup != 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        CountPart cp;
        cp.heads = wh[0] + wh[1] + wh[2] + wh[3];
        cp.dup = wd[0] | wd[1] | wd[2] | wd[3];
        part[blockIdx.x] = cp;
    }
}

// Size the brick table from the count (load <= 1/2, at least 2^10 slots, at
// most the workspace's 2^max_log2) and mark its slots empty.  Every workgroup
// sums the kCountBlocks partials itself.
__global__ void __launch_bounds__(256) k_brick_fill(BrickSlot* table, int max_log2,
                                                    const CountPart* __restrict__ part,
                                                    BuildFlags* flags) {
    __shared__ uint32_t wh[4];
    const int t = threadIdx.x;
    uint32_t nb = 0;
    for (int b = t; b < kCountBlocks; b += 256) nb += part[b].heads;
    for (int o = 32; o > 0; o >>= 1) nb += __shfl_xor(nb, o);
    if ((t & 63) == 0) wh[t >> 6] = nb;
    __syncthreads();
    nb = wh[0] + wh[1] + wh[2] + wh[3];
    int L = ceil_log2_dev(2u * nb);
    L = L < 10 ? 10 : (L > max_log2 ? max_log2 : L);
    if (blockIdx.x == 0 && t == 0) {
        flags->log2_bricks = (uint32_t)L;
        flags->nbricks = nb;
    }
    const int64_t cap = (int64_t)1 << L;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + t; i < cap; i += (int64_t)gridDim.x * blockDim.x)
        table[i].key = kEmptyKey;
}

__device__ __forceinline__ unsigned long long shfl_down64(unsigned long long v, int o) {
    const uint32_t lo = (uint32_t)__shfl_down((int)(uint32_t)v, o);
    const uint32_t hi = (uint32_t)__shfl_down((int)(uint32_t)(v >> 32), o);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long shfl_up64(unsigned long long v, int o) {
    const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, o);
    const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), o);
    return ((unsigned long long)hi << 32) | lo;
}

// Insert every brick: a wave takes 64 consecutive sorted codes, ORs the cell
// bits of each run of equal brick keys with a segmented suffix scan across its
// lanes, and the first voxel of each run inserts (brick key -> first position,
// cell mask).  A run that goes on past the wave's last lane is finished by its
// head reading on.
__global__ void __launch_bounds__(256) k_brick_insert(const uint64_t* __restrict__ codes, int64_t N,
                                                      BrickSlot* table, const BuildFlags* flags) {
    const int L = (int)flags->log2_bricks;
    const uint32_t cap_mask = (1u << L) - 1u;
    const int lane = threadIdx.x & 63;
    const int64_t wstride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63); base < N; base += wstride) {
        const int64_t i = base + lane;
        const bool act = i < N;
        const uint64_t c = act ? codes[i] : ~0ull;
        const unsigned long long key = c >> 6;   // ~0 >> 6 is above every real brick key
        unsigned long long m = act ? 1ull << (c & 63u) : 0ull;
        unsigned long long prev = shfl_up64(key, 1);
        if (lane == 0) prev = (i > 0) ? (codes[i - 1] >> 6) : ~0ull;
        const bool head = act && key != prev;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long om = shfl_down64(m, o);
            const unsigned long long ok = shfl_down64(key, o);
            if (lane + o < 64 && ok == key) m |= om;
        }
        const unsigned long long last =                                  // lane 63's key
            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), 63) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, 63);
        if (head) {
            if (key == last) {
                for (int64_t j = base + 64; j < N; ++j) {
                    const uint64_t cj = codes[j];
                    if ((cj >> 6) != key) break;
                    m |= 1ull << (cj & 63u);
                }
            }
            uint32_t s = brick_home(key, L);
            for (;;) {  // terminates: load <= 1/2 leaves empty slots and the probe is linear
                const unsigned long long prevk = atomicCAS(&table[s].key, kEmptyKey, key);
                if (prevk == kEmptyKey || prevk == key) {
                    table[s].start = (uint32_t)i;
                    table[s].mask = m;
                    break;
                }
                s = (s + 1) & cap_mask;
            }
        }
    }
}

// One workgroup: the map's valid-pair count from the per-tile counts, and the
// duplicate flag from the brick-count partials (when building).  The results
// go to the map's header and, when building, to the host-visible flags.
constexpr int kFinishThreads = 1024;
__global__ void __launch_bounds__(kFinishThreads) k_finish(const unsigned long long* __restrict__ tile_pairs,
                                                           const uint32_t* __restrict__ dcount,
                                                           int64_t ntiles, int64_t ndist,
                                                           const CountPart* __restrict__ cpart,
                                                           MapInfo* info, BuildFlags* hflags) {
    __shared__ unsigned long long ws[kFinishThreads / 64];
    __shared__ uint32_t wd[kFinishThreads / 64];
    __shared__ uint32_t wm[kFinishThreads / 64];
    const int t = threadIdx.x;
    unsigned long long v = 0;
    uint32_t dmax = 0;
    const int64_t nmax = ntiles > ndist ? ntiles : ndist;
    for (int64_t i0 = t; i0 < nmax; i0 += 4 * kFinishThreads) {
        unsigned long long x[4];
        uint32_t d[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // four independent loads in flight
            const int64_t i = i0 + (int64_t)u * kFinishThreads;
            x[u] = i < ntiles ? tile_pairs[i] : 0;
            uint32_t dv = i < ndist ? dcount[i] : 0u;
            if (dv != kNoDistinct && (dv & kLayerPasses))   // three passes: their rows together
                dv = (uint32_t)(layer_rows(dv, 0) + layer_rows(dv, 1) + layer_rows(dv, 2));
            d[u] = dv;
        }
        v += x[0] + x[1] + x[2] + x[3];
        dmax = max(dmax, max(max(d[0], d[1]), max(d[2], d[3])));
    }
    for (int o = 32; o > 0; o >>= 1) dmax = max(dmax, (uint32_t)__shfl_xor((int)dmax, o));
    uint32_t dup = 0;
    if (cpart)
        for (int b = t; b < kCountBlocks; b += kFinishThreads) dup |= cpart[b].dup;
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
        v += ((unsigned long long)hi << 32) | lo;
    }
    const uint64_t anydup = __ballot(dup != 0);
    if ((t & 63) == 0) {
        ws[t >> 6] = v;
        wd[t >> 6] = anydup != 0;
        wm[t >> 6] = dmax;
    }
    __syncthreads();
    if (t == 0) {
        unsigned long long tot = 0;
        uint32_t d = 0, m = 0;
        for (int w = 0; w < kFinishThreads / 64; ++w) {
            tot += ws[w];
            d |= wd[w];
            m = max(m, wm[w]);
        }
        info->valid_pairs = tot;
        info->max_distinct = m;
        if (hflags) {
            hflags->valid_pairs = tot;
            hflags->duplicate = d;
            hflags->max_distinct = m;
        }
    }
}

// Distinct neighbour rows of one half tile (kDistinctRows rows of the
// schedule, one workgroup each), for one staging pass or, past the cap, for
// three passes of one offset layer each.  A pass puts the caller indices of
// the present neighbours at its offsets into an LDS hash set, each (row,
// offset) remembering the hash slot of its neighbour; if there are at most
// kDistinctCap distinct ones, the occupied hash slots are numbered in table
// order (a workgroup prefix sum), the distinct rows are listed in that order,
// and each (row, offset) gets the code of its neighbour's number (the slot
// map assembled in LDS, then written with 16-byte stores).  Which number a
// row gets can differ from run to run (the probe order of colliding keys
// does); the forward reads the same values whatever the numbering.
constexpr int kDistinctHashBits = 11;
constexpr int kDistinctHash = 1 << kDistinctHashBits;
constexpr int kDistinctProbe = 64;
constexpr uint32_t kHashEmpty = 0xFFFFFFFFu;
static_assert(kDistinctCap < kDistinctHash / 4, "hash load");

__global__ void __launch_bounds__(kDistinctRows) k_tile_distinct(const int32_t* __restrict__ nbr_m, int64_t N,
                                                                 int64_t Npad, int K, uint32_t* __restrict__ dcount,
                                                                 int32_t* __restrict__ drow,
                                                                 uint16_t* __restrict__ smap) {
    constexpr int R = kDistinctRows;
    __shared__ uint32_t hkey[kDistinctHash];   // keys; after the numbering, each key's rank
    // per (offset, row): the hash slot of the row's neighbour during a pass,
    // then its slot code
    __shared__ __attribute__((aligned(16))) uint16_t smt[kDistinctMaxK * R];
    __shared__ uint32_t over;
    __shared__ uint32_t wsum[R / 64];
    const int t = threadIdx.x;
    const int64_t half = blockIdx.x;
    const int64_t row = half * R + t;
    const uint32_t N32 = (uint32_t)N;
    if (K > kDistinctMaxK) {   // no slot maps for such maps
        if (t == 0) dcount[half] = kNoDistinct;
        return;
    }
    auto home = [](uint32_t p) -> uint32_t { return (p * 2654435761u) >> (32 - kDistinctHashBits); };
    uint32_t pk[kDistinctMaxK];
#pragma unroll
    for (int k = 0; k < kDistinctMaxK; ++k) {
        const uint32_t m = k < K ? (uint32_t)nbr_m[(int64_t)k * Npad + row] : N32;
        pk[k] = m < N32 ? m : kHashEmpty;
    }
    const int lane = t & 63, wv = t >> 6;
    const int pos = slot_pos(t);
    // One staging pass over offsets [klo, khi): its rows listed at dr, the
    // codes of its offsets into smt.  Returns the row count, or -1 over the
    // cap (uniform).
    auto pass = [&](int klo, int khi, int32_t* dr) -> int {
        __syncthreads();   // the previous pass's table is read
        for (int i = t; i < kDistinctHash; i += R) hkey[i] = kHashEmpty;
        if (t == 0) over = 0;
        __syncthreads();
        // Insert, keeping each offset's hash slot in smt (kDistinctHash: missing):
        // one compare-and-swap per probed slot (it both finds the key and
        // claims an empty slot; a read before it cost 20% more).  A probe of
        // more than kDistinctProbe slots (a table filling up: far more
        // distinct rows than the cap) gives up and marks the pass as over the
        // cap, so every probe ends; the count is taken afterwards, without a
        // shared counter in the insert loop.
#pragma unroll
        for (int k = 0; k < kDistinctMaxK; ++k) {
            if (k < klo || k >= khi) continue;
            uint32_t h = kDistinctHash;
            if (pk[k] != kHashEmpty) {
                const uint32_t p = pk[k];
                h = home(p);
                int probes = 0;
                for (;;) {
                    const uint32_t prev = atomicCAS(&hkey[h], kHashEmpty, p);
                    if (prev == kHashEmpty || prev == p) break;
                    if (++probes > kDistinctProbe) {
                        over = 1;
                        break;
                    }
                    h = (h + 1) & (kDistinctHash - 1);
                }
            }
            smt[k * R + pos] = (uint16_t)h;
        }
        __syncthreads();
        if (over) return -1;
        // number the occupied slots (thread t owns slots SPT t .. SPT t +
        // SPT - 1) with a workgroup prefix sum of the per-thread counts
        constexpr int SPT = kDistinctHash / R;
        int c = 0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) c += hkey[SPT * t + i] != kHashEmpty;
        int incl = c;
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wv] = (uint32_t)incl;
        __syncthreads();
        int off = incl - c;
        for (int v = 0; v < wv; ++v) off += (int)wsum[v];
        uint32_t n = 0;
        for (int v = 0; v < R / 64; ++v) n += wsum[v];
        if (n > (uint32_t)kDistinctCap) return -1;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const uint32_t m = hkey[SPT * t + i];
            if (m != kHashEmpty) {
                hkey[SPT * t + i] = (uint32_t)off;   // (only this thread reads this slot here)
                dr[off++] = (int32_t)m;
            }
        }
        __syncthreads();
        // slot code of every (row, offset) of the pass: thread t = row t
#pragma unroll
        for (int k = 0; k < kDistinctMaxK; ++k) {
            if (k < klo || k >= khi) continue;
            const uint32_t h = smt[k * R + pos];
            const uint32_t slot = h < (uint32_t)kDistinctHash ? hkey[h] : (uint32_t)kDistinctCap;
            smt[k * R + pos] = (uint16_t)slot_code(slot);
        }
        return (int)n;
    };
    int32_t* dr = drow + half * kDistinctListCap;
    uint32_t code = kNoDistinct;
    const int n = pass(0, K, dr);
    if (n >= 0) {
        code = (uint32_t)n;
    } else if (K == 9 * kDistinctLayers) {
        // three passes, one per layer of nine offsets
        uint32_t c3 = kLayerPasses;
        int p = 0;
        for (; p < kDistinctLayers; ++p) {
            const int np = pass(9 * p, 9 * p + 9, dr + kDistinctCap * p);
            if (np < 0) break;
            c3 |= (uint32_t)np << (10 * p);
        }
        if (p == kDistinctLayers) code = c3;
    }
    if (code == kNoDistinct) {   // uniform
        if (t == 0) dcount[half] = kNoDistinct;
        return;
    }
    __syncthreads();
    uint4* sm = (uint4*)(smap + half * (int64_t)K * R);
    const uint4* src = (const uint4*)smt;
    for (int i = t; i < K * R / 8; i += R) sm[i] = src[i];
    if (t == 0) dcount[half] = code;
}

// ---------------------------------------------------------------------------
// LSD radix sort, 8-bit digits.  Block b owns elements [b*4096, (b+1)*4096);
// wave w of its 16 owns the 256 elements [b*4096 + w*256, ...), taken 64 at a
// time in order, so (wave, round, lane) is the input order and each pass is
// stable.  hist layout: hist[d * nblk + b] (digit-major).  The first pass's
// histogram comes from k_pack.
// ---------------------------------------------------------------------------
constexpr int kWaveItems = kSortChunk / (kSortThreads / 64) / 64;   // rounds per wave (4)

__global__ void __launch_bounds__(kSortThreads) k_radix_hist(const uint64_t* __restrict__ codes,
                                                             int64_t N, int shift,
                                                             uint32_t* __restrict__ hist,
                                                             int64_t nblk) {
    __shared__ uint32_t h[kRadix];
    const int t = threadIdx.x;
    if (t < kRadix) h[t] = 0;
    const int64_t base = (int64_t)blockIdx.x * kSortChunk;
    uint32_t d[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = base + (int64_t)r * kSortThreads + t;
        d[r] = e < N ? (uint32_t)(codes[e] >> shift) & (kRadix - 1) : kRadix;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortItems; ++r)
        if (d[r] < kRadix) atomicAdd(&h[d[r]], 1u);
    __syncthreads();
    if (t < kRadix) hist[(int64_t)t * nblk + blockIdx.x] = h[t];
}

// Exclusive scan of each digit's row hist[d*nblk .. d*nblk+nblk) in place;
// totals[d] = the row's sum.  One block per digit.  On the first pass
// (ppart != NULL) block 0 also ORs the pack partials into the host-visible
// flags (the Morton bits that vary, and the range check).
__global__ void __launch_bounds__(256) k_radix_rowscan(uint32_t* __restrict__ hist, int64_t nblk,
                                                       uint32_t* __restrict__ totals,
                                                       const PackPart* __restrict__ ppart,
                                                       BuildFlags* hflags) {
    __shared__ uint32_t part[256];
    __shared__ uint64_t wor[4];
    __shared__ uint32_t wbad[4];
    const int t = threadIdx.x;
    if (ppart && blockIdx.x == 0) {
        uint64_t x = 0;
        uint32_t bad = 0;
        for (int64_t b = t; b < nblk; b += 256) {
            x |= ppart[b].xor_or;
            bad |= ppart[b].bad;
        }
        x = wave_or(x);
        const uint64_t anybad = __ballot(bad != 0);
        if ((t & 63) == 0) {
            wor[t >> 6] = x;
            wbad[t >> 6] = anybad != 0;
        }
        __syncthreads();
        if (t == 0) {
            hflags->morton_xor_or = wor[0] | wor[1] | wor[2] | wor[3];
            hflags->range_error = wbad[0] | wbad[1] | wbad[2] | wbad[3];
        }
    }
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

// Scatter one pass.  Each wave ranks its elements among equal digits with
// ballots (a lane's peers are the lanes whose 8 digit bits all agree with its
// own) and a wave-private running count per digit in LDS; a wave's LDS
// operations complete in order, so no barrier is needed between rounds.  The
// block's elements are then placed in LDS in sorted order (digit, wave, rank)
// and written out from there: consecutive lanes hold consecutive elements of
// a digit's run, so the global writes come in contiguous runs rather than one
// element per cache line.
__global__ void __launch_bounds__(kSortThreads) k_radix_scatter(
    const uint64_t* __restrict__ codes_in, const uint32_t* __restrict__ idx_in, int64_t N, int shift,
    const uint32_t* __restrict__ hist, int64_t nblk, const uint32_t* __restrict__ totals,
    uint64_t* __restrict__ codes_out, uint32_t* __restrict__ idx_out) {
    constexpr int NW = kSortThreads / 64;
    __shared__ uint32_t cnt[NW][kRadix];
    __shared__ uint32_t scan[kRadix];
    __shared__ int32_t gdelta[kRadix];               // global position - block-local position, per digit
    __shared__ uint64_t lcode[kSortChunk];
    __shared__ uint32_t lid[kSortChunk];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = t >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kSortChunk;
    const int64_t w0 = b0 + (int64_t)wv * (kWaveItems * 64);
    const int nloc = (int)(N - b0 < kSortChunk ? N - b0 : kSortChunk);   // elements of this block
    uint64_t code[kWaveItems];
    uint32_t id[kWaveItems];
#pragma unroll
    for (int r = 0; r < kWaveItems; ++r) {
        const int64_t e = w0 + r * 64 + lane;
        code[r] = e < N ? codes_in[e] : 0;
        id[r] = e < N ? idx_in[e] : 0;
    }
#pragma unroll
    for (int i = 0; i < kRadix / 64; ++i) cnt[wv][lane + 64 * i] = 0;
    // digit start = exclusive scan of the totals (thread t < kRadix: digit t)
    const bool dt = t < kRadix;
    const uint32_t tot = dt ? totals[t] : 0u;
    if (dt) scan[t] = tot;
    __syncthreads();
    for (int o = 1; o < kRadix; o <<= 1) {
        const uint32_t v = (dt && t >= o) ? scan[t - o] : 0;
        __syncthreads();
        if (dt) scan[t] += v;
        __syncthreads();
    }
    const uint32_t blockbase = dt ? scan[t] - tot + hist[(int64_t)t * nblk + blockIdx.x] : 0u;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t rank[kWaveItems];
#pragma unroll
    for (int r = 0; r < kWaveItems; ++r) {
        const bool act = w0 + r * 64 + lane < N;
        const uint32_t d = (uint32_t)(code[r] >> shift) & (kRadix - 1);
        uint64_t peers = __ballot(act);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const uint32_t below = __popcll(peers & lt_mask);
        const uint32_t c = cnt[wv][d];
        rank[r] = c + below;
        if (act && below == 0) cnt[wv][d] = c + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    // block-local layout: digit-major, then wave; thread t < kRadix owns digit t
    uint32_t dcount = 0;
    if (dt) {
#pragma unroll
        for (int w = 0; w < NW; ++w) dcount += cnt[w][t];
        scan[t] = dcount;
    }
    __syncthreads();
    for (int o = 1; o < kRadix; o <<= 1) {
        const uint32_t v = (dt && t >= o) ? scan[t - o] : 0;
        __syncthreads();
        if (dt) scan[t] += v;
        __syncthreads();
    }
    if (dt) {
        const uint32_t lstart = scan[t] - dcount;
        gdelta[t] = (int32_t)(blockbase - lstart);
        uint32_t run = lstart;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t c = cnt[w][t];
            cnt[w][t] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kWaveItems; ++r) {
        if (w0 + r * 64 + lane < N) {
            const uint32_t d = (uint32_t)(code[r] >> shift) & (kRadix - 1);
            const uint32_t lp = cnt[wv][d] + rank[r];
            lcode[lp] = code[r];
            lid[lp] = id[r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int e = t + r * kSortThreads;
        if (e < nloc) {
            const uint64_t c = lcode[e];
            const int64_t pos = (int64_t)e + gdelta[(uint32_t)(c >> shift) & (kRadix - 1)];
            codes_out[pos] = c;
            idx_out[pos] = lid[e];
        }
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
    unsigned long long* tile_pairs;   // per-tile count of present (row, offset) pairs
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
template <bool LEAN = false>
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
    if constexpr (LEAN) {
        // one brick at a time (a rarely taken path kept out of the caller's
        // register budget)
#pragma unroll 1
        for (int i = 0; i < 8; ++i) {
            const unsigned long long k1[1] = {key[i]};
            const bool w1[1] = {true};
            uint32_t s1[1];
            unsigned long long m1[1];
            find_bricks<1>(a.table, L, k1, w1, s1, m1);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q == i) {
                    st[q] = s1[0];
                    mk[q] = m1[0];
                }
        }
    } else {
        find_bricks<8>(a.table, L, key, want, st, mk);
    }
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

// ---------------------------------------------------------------------------
// Stable sort of a tile's 256 (key, row) pairs by key: LSD radix with 7-bit
// digits, one element per thread.  Each wave ranks its 64 keys among equal
// digits with ballots; the digit totals of the four waves are scanned (digit
// major, then wave) to place every element; positions follow (wave, lane), so
// each pass is stable.  On return rowsrc[i] is the row at sorted position i
// (visible to the workgroup).
// ---------------------------------------------------------------------------
constexpr int kSortDigitBits = 7;
constexpr int kSortDigits = 1 << kSortDigitBits;

struct TileSortLds {
    uint32_t key[kTileRows];
    int32_t item[kTileRows];
    uint32_t cnt[kTileRows / 64][kSortDigits];
};

__device__ void tile_radix_sort(uint32_t key, int passes, TileSortLds& s, int32_t* rowsrc) {
    constexpr int NW = kTileRows / 64, DPL = kSortDigits / 64;   // digits per lane
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int32_t item = t;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int p = 0; p < passes; ++p) {
#pragma unroll
        for (int i = 0; i < DPL; ++i) s.cnt[wv][lane * DPL + i] = 0;   // this wave's row only
        const uint32_t dg = (key >> (kSortDigitBits * p)) & (kSortDigits - 1);
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < kSortDigitBits; ++b) {
            const bool bit = (dg >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const uint32_t below = __popcll(peers & lt);
        if (below == 0) s.cnt[wv][dg] = __popcll(peers);
        __syncthreads();
        // every wave scans the (digit, wave) counts itself: lane l covers
        // digits DPL*l .. DPL*l + DPL-1; this wave's base of digit e is the
        // count of all smaller digits plus this digit's count in lower waves
        uint32_t tot[DPL], mine[DPL];
        uint32_t run = 0;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const int e = lane * DPL + i;
            tot[i] = 0;
            mine[i] = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint32_t c = s.cnt[w][e];
                tot[i] += c;
                if (w < wv) mine[i] += c;
            }
            run += tot[i];
        }
        uint32_t inc = run;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t v = (uint32_t)__shfl_up((int)inc, o);
            if (lane >= o) inc += v;
        }
        uint32_t b = inc - run;
        uint32_t base[DPL];
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            base[i] = b + mine[i];
            b += tot[i];
        }
        // digit dg's base is entry dg % DPL of lane dg / DPL
        uint32_t bsel = 0;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const uint32_t bi = (uint32_t)__shfl((int)base[i], (int)(dg / DPL));
            if ((int)(dg % DPL) == i) bsel = bi;
        }
        const uint32_t pos = bsel + below;
        s.key[pos] = key;
        s.item[pos] = item;
        __syncthreads();
        key = s.key[t];
        item = s.item[t];
    }
    rowsrc[t] = item;
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Tile query for the 3x3x3 stencil at dilation <= 2 (mode 0).  A row's 27
// neighbours lie in the 8 bricks (c0|c1)^3; the tile's rows share most of
// them (about 90 distinct bricks for 256 surface rows).  The rows insert
// their brick keys into an LDS hash set and each distinct brick is probed in
// the global table once; a row then finds its bricks' cell masks and first
// positions in LDS.  A tile with more distinct bricks than the set holds
// takes the per-row path (every row probes its 8 bricks in the global table).
// The rows' validity masks come from the cell masks alone; the rows are
// sorted by mask, and then each thread takes the row at its sorted position
// and writes that row's 27 caller indices (no per-tile buffer of them).
// ---------------------------------------------------------------------------
constexpr int kQHashBits = 9;
constexpr int kQHS = 1 << kQHashBits;       // LDS hash slots
constexpr int kQProbe = 32;                 // longest LDS probe sequence before the per-row path

__device__ __forceinline__ uint32_t lds_home(unsigned long long key) {
    return (uint32_t)((key * 0xC2B2AE3D27D4EB4Full) >> (64 - kQHashBits));
}

// Present neighbours of a row (biased coordinates u, dilation d <= 2) at the
// 27 offsets, from the cell masks bm and first sorted positions bb of its 8
// bricks (c0|c1)^3 (index: x, y, z bit = upper brick): returns the validity
// mask (bit k); with VALUES also the caller indices (N where missing).
template <bool VALUES>
__device__ __forceinline__ uint32_t row27(const QueryArgs& a, const uint32_t (&u)[3],
                                          const unsigned long long (&bm)[8], const uint32_t (&bb)[8],
                                          int32_t (&v)[27]) {
    const uint32_t d = (uint32_t)a.dilation;
    const uint32_t top = 2u * (uint32_t)kCoordBias;
    const int32_t N32 = (int32_t)a.N;
    // per axis and offset o = -1, 0, +1: in range, neighbour in the upper
    // brick (c1) rather than c0, and its two low coordinate bits placed as in
    // the cell index
    bool okv[3][3], upv[3][3];
    uint32_t part[3][3];
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
        const bool lo_ok = u[ax] >= d, hi_ok = u[ax] + d < top;
        const uint32_t c0 = (lo_ok ? u[ax] - d : u[ax]) >> 2;
        const uint32_t c1 = (hi_ok ? u[ax] + d : u[ax]) >> 2;
        const uint32_t nv[3] = {u[ax] - d, u[ax], u[ax] + d};
        okv[ax][0] = lo_ok;
        okv[ax][1] = true;
        okv[ax][2] = hi_ok;
        upv[ax][0] = false;
        upv[ax][1] = (u[ax] >> 2) != c0;
        upv[ax][2] = c1 != c0;
#pragma unroll
        for (int o = 0; o < 3; ++o) part[ax][o] = ((nv[o] & 1u) << (2 - ax)) | ((nv[o] & 2u) << (4 - ax));
    }
    // the brick of offset (ox, oy, oz) is combo (up_x, up_y, up_z): select
    // along x, then y, then z
    uint32_t mask = 0;
#pragma unroll
    for (int ox = 0; ox < 3; ++ox) {
        unsigned long long mx[4];
        uint32_t bx[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            mx[q] = upv[0][ox] ? bm[4 + q] : bm[q];
            bx[q] = upv[0][ox] ? bb[4 + q] : bb[q];
        }
#pragma unroll
        for (int oy = 0; oy < 3; ++oy) {
            unsigned long long my[2];
            uint32_t by[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                my[r] = upv[1][oy] ? mx[2 + r] : mx[r];
                by[r] = upv[1][oy] ? bx[2 + r] : bx[r];
            }
#pragma unroll
            for (int oz = 0; oz < 3; ++oz) {
                const unsigned long long m8 = upv[2][oz] ? my[1] : my[0];
                const bool ok = okv[0][ox] && okv[1][oy] && okv[2][oz];
                const uint32_t cell = part[0][ox] | part[1][oy] | part[2][oz];
                const bool present = ok && ((m8 >> cell) & 1ull);
                const int k = 9 * ox + 3 * oy + oz;
                mask |= (present ? 1u : 0u) << k;
                if constexpr (VALUES) {
                    int32_t r = N32;
                    if (present) {
                        const uint32_t b8 = upv[2][oz] ? by[1] : by[0];
                        r = (int32_t)a.morton_idx[b8 + (uint32_t)__popcll(m8 & ((1ull << cell) - 1ull))];
                    }
                    v[k] = r;
                }
            }
        }
    }
    return mask;
}

// (A bound of four workgroups per CU: the kernel's 95 VGPRs still give five,
// and under a bound of five the compiler moves 80 bytes per lane to scratch.)
__global__ void __launch_bounds__(kTileRows, 4) k_tile_query27(QueryArgs a) {
    __shared__ unsigned long long hkey[kQHS];
    __shared__ unsigned long long hmask[kQHS];
    __shared__ uint32_t hstart[kQHS];
    __shared__ TileSortLds srt;
    __shared__ int32_t caller[kTileRows];
    __shared__ __attribute__((aligned(16))) int32_t rowsrc[kTileRows];
    __shared__ unsigned long long rcode[kTileRows];                        // each row's Morton code
    __shared__ __attribute__((aligned(16))) uint16_t rslot[kTileRows][8];   // its bricks' LDS slots
    __shared__ uint32_t bmk[27];                                           // block masks, sorted rows
    __shared__ uint32_t q_over;
    __shared__ unsigned long long cnt_s[kTileRows / 64];

    const int t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int64_t tile = blockIdx.x;
    const int64_t j = tile * kTileRows + t;
    const int32_t N32 = (int32_t)a.N;

    int64_t n = -1;
    uint32_t u[3] = {0u, 0u, 0u};   // biased coordinates
    uint64_t code = 0;
    if (j < a.N) {
        n = (int64_t)a.morton_idx[j];
        code = a.codes[j];
        u[0] = compact3(code >> 2);
        u[1] = compact3(code >> 1);
        u[2] = compact3(code);
    }
    caller[t] = (int32_t)n;
    rcode[t] = code;
    for (int q = t; q < kQHS; q += kTileRows) hkey[q] = kEmptyKey;
    if (t < 27) bmk[t] = 0;
    if (t == 0) q_over = 0;
    __syncthreads();

    const int L = (int)a.bflags->log2_bricks;
    const uint32_t d = (uint32_t)a.dilation;
    const uint32_t top = 2u * (uint32_t)kCoordBias;
    bool lo_ok[3], hi_ok[3];
    uint32_t c0[3], c1[3];
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
        lo_ok[ax] = u[ax] >= d;
        hi_ok[ax] = u[ax] + d < top;
        c0[ax] = (lo_ok[ax] ? u[ax] - d : u[ax]) >> 2;
        c1[ax] = (hi_ok[ax] ? u[ax] + d : u[ax]) >> 2;
    }
    // insert the row's 8 brick keys into the LDS set; slot[i] = where key i
    // lives.  Consecutive rows mostly share their bricks, so only the first
    // lane of each run of equal keys inserts, and the run takes its slot.
    // (Padding rows, n < 0, are the last rows of the last tile.)  All eight
    // home-slot compare-and-swaps go out together; the few collisions then
    // probe on.  A key not placed within kQProbe slots sends the tile to the
    // per-row path, which is always correct.
    // brick key = spread(bz) | spread(by) << 1 | spread(bx) << 2, from the two
    // brick coordinates of each axis
    unsigned long long sp[3][2];
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
        sp[ax][0] = spread3(c0[ax]) << (2 - ax);
        sp[ax][1] = c1[ax] == c0[ax] ? sp[ax][0] : spread3(c1[ax]) << (2 - ax);
    }
    unsigned long long key[8];
    bool head[8], placed[8];
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        key[i] = sp[0][(i >> 2) & 1] | sp[1][(i >> 1) & 1] | sp[2][i & 1];
        const unsigned long long prevkey = shfl_up64(key[i], 1);
        head[i] = n >= 0 && (lane == 0 || prevkey != key[i]);
        q[i] = lds_home(key[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        placed[i] = true;
        if (head[i]) {
            const unsigned long long prev = atomicCAS(&hkey[q[i]], kEmptyKey, key[i]);
            placed[i] = prev == kEmptyKey || prev == key[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!placed[i]) {
            for (int probe = 1; probe < kQProbe; ++probe) {
                q[i] = (q[i] + 1) & (kQHS - 1);
                const unsigned long long prev = atomicCAS(&hkey[q[i]], kEmptyKey, key[i]);
                if (prev == kEmptyKey || prev == key[i]) {
                    placed[i] = true;
                    break;
                }
            }
            if (!placed[i]) q_over = 1u;
        }
    }
    uint32_t slot[8];
    const uint64_t upto_me = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint64_t heads = __ballot(head[i]) & upto_me;
        const int src = heads ? 63 - __builtin_clzll(heads) : lane;
        slot[i] = (uint32_t)__shfl((int)q[i], src);
    }
    {
        u32x4 sl;
#pragma unroll
        for (int i = 0; i < 4; ++i) sl[i] = (slot[2 * i] & 0xFFFFu) | (slot[2 * i + 1] << 16);
        *(u32x4*)&rslot[t][0] = sl;
    }
    __syncthreads();
    const bool over = q_over != 0u;

    // each distinct brick is probed once: thread t takes slots 2t and 2t+1
    if (!over) {
        unsigned long long k2[2];
        bool want[2];
        uint32_t st[2];
        unsigned long long mk[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            k2[r] = hkey[2 * t + r];
            want[r] = k2[r] != kEmptyKey;
        }
        find_bricks<2>(a.table, L, k2, want, st, mk);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            hmask[2 * t + r] = mk[r];
            hstart[2 * t + r] = st[r];
        }
    }
    __syncthreads();

    // the row's validity mask (the cell masks only; the per-row path probes
    // the global table)
    uint32_t mask = 0;
    if (n >= 0) {
        int32_t v[27];
        if (over) {
            neighbours27<true>(a, L, (int)u[0] - kCoordBias, (int)u[1] - kCoordBias, (int)u[2] - kCoordBias, v);
#pragma unroll
            for (int k = 0; k < 27; ++k) mask |= (v[k] != N32 ? 1u : 0u) << k;
        } else {
            unsigned long long bm[8];
            uint32_t bb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bm[i] = hmask[slot[i]];
                bb[i] = 0;
            }
            mask = row27<false>(a, u, bm, bb, v);
        }
    }
    unsigned long long cnt = (unsigned long long)__popc(mask);
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) cnt_s[wv] = cnt;
    __syncthreads();
    if (t == 0) a.tile_pairs[tile] = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];

    // rows by validity mask inside each half tile: the half is the key's top
    // bit; a padding row (only after all real rows) takes the all-ones mask,
    // so the stable sort keeps it behind every real row of its half
    static_assert(kTileRows == 2 * kSortRows && 27 + 1 <= 4 * kSortDigitBits, "sort key");
    tile_radix_sort(((uint32_t)(t / kSortRows) << 27) | (n < 0 ? (1u << 27) - 1u : mask), 4, srt, rowsrc);

    // thread t takes the row at sorted position t: its caller index, its 27
    // neighbours (one coalesced store per offset) and its bits of the 16-row
    // block masks
    const int64_t row0 = tile * kTileRows;
    const int src = rowsrc[t];
    const int32_t ns = caller[src];
    a.order[row0 + t] = ns;
    int32_t v[27];
    if (ns < 0) {
#pragma unroll
        for (int k = 0; k < 27; ++k) v[k] = N32;
    } else {
        const uint64_t cs = rcode[src];
        const uint32_t us[3] = {compact3(cs >> 2), compact3(cs >> 1), compact3(cs)};
        if (over) {
            neighbours27<true>(a, L, (int)us[0] - kCoordBias, (int)us[1] - kCoordBias, (int)us[2] - kCoordBias, v);
        } else {
            const u32x4 sl = *(const u32x4*)&rslot[src][0];
            unsigned long long bm[8];
            uint32_t bb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t q8 = (sl[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                bm[i] = hmask[q8];
                bb[i] = hstart[q8];
            }
            (void)row27<true>(a, us, bm, bb, v);
        }
    }
#pragma unroll
    for (int k = 0; k < 27; ++k) {
        a.nbr_m[(int64_t)k * a.Npad + row0 + t] = v[k];
        const uint64_t bal = __ballot(v[k] != N32);
        uint32_t m4 = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) m4 |= (((bal >> (16 * b)) & 0xFFFFull) != 0ull ? 1u : 0u) << b;
        if (lane == 0 && m4) atomicOr(&bmk[k], m4 << (4 * wv));
    }
    __syncthreads();
    static_assert(kBlocksPerTile == 4 * (kTileRows / 64), "four 16-row blocks per wave");
    if (t < 27) a.blkmask[tile * 27 + t] = (uint16_t)bmk[t];
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
    if (t == 0) a.tile_pairs[tile] = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
    // stable rank of this row's key inside its half tile: each wave sorts its
    // 64 (key, row) pairs, and a row's rank is the number of pairs before it in
    // the two sorted runs of its half (binary searches)
    const unsigned long long my = keys[t];
    {
        unsigned long long sk = my;
        uint32_t si = (uint32_t)t;
        wave_sort64(sk, si, lane);
        run_k[t] = sk;
        run_i[t] = si;
    }
    __syncthreads();
    static_assert(kSortRows % 64 == 0, "whole waves per half tile");
    constexpr int WPH = kSortRows / 64;      // waves per half tile
    const int hw0 = (wv / WPH) * WPH;        // first wave of this row's half
    int rank = hw0 * 64;
#pragma unroll
    for (int w3 = 0; w3 < WPH; ++w3) {
        const int b0 = (hw0 + w3) * 64;
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

hipError_t run_tile_query(QueryArgs qa, const ArenaLayout& al, hipStream_t stream) {
    if (qa.mode == 0 && qa.side == 3 && qa.dilation <= 2)
        k_tile_query27<<<dim3((unsigned)al.ntiles), dim3(kTileRows), 0, stream>>>(qa);
    else
        k_tile_query<<<dim3((unsigned)al.ntiles), dim3(kTileRows), 0, stream>>>(qa);
    return hipGetLastError();
}

}  // namespace

int batch_slab_log2(int batches) {
    int l = 0;
    while (batches > 1 && (1 << l) < batches) ++l;
    return l;
}

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
    l.pairs_off = off;
    off = align_up(off + (size_t)8 * l.ntiles, 256);
    l.info_off = off;
    off = align_up(off + sizeof(MapInfo), 256);
    l.dcount_off = off;
    off = align_up(off + (size_t)4 * kDistinctPerTile * l.ntiles, 256);
    l.drow_off = off;
    off = align_up(off + (K <= kDistinctMaxK ? (size_t)4 * kDistinctListCap * kDistinctPerTile * l.ntiles : 0), 256);
    l.smap_off = off;
    off = align_up(off + (K <= kDistinctMaxK ? (size_t)2 * K * kTileRows * l.ntiles : 0), 256);
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
    l.pack_part = off;
    off = align_up(off + sizeof(PackPart) * (size_t)l.nsort_blocks, 256);
    l.count_part = off;
    off = align_up(off + sizeof(CountPart) * (size_t)kCountBlocks, 256);
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

namespace {

// Host-visible flags: pinned, coherent host memory that the kernels write
// directly, so reading them needs no copy.  One buffer per host thread (a build
// runs on its caller's thread and is finished when it returns), kept until the
// process ends.  Returns the host pointer; *dev receives the device address.
BuildFlags* host_flags_buffer(BuildFlags** dev) {
    thread_local BuildFlags* h = nullptr;
    thread_local BuildFlags* d = nullptr;
    if (!h) {
        void* q = nullptr;
        if (hipHostMalloc(&q, sizeof(BuildFlags), hipHostMallocCoherent | hipHostMallocPortable) != hipSuccess) return nullptr;
        void* qd = nullptr;
        if (hipHostGetDevicePointer(&qd, q, 0) != hipSuccess) {
            (void)hipHostFree(q);
            return nullptr;
        }
        h = (BuildFlags*)q;
        d = (BuildFlags*)qd;
    }
    *dev = d;
    return h;
}

// One completion event per host thread and device (the stream's), created on
// first use.
hipEvent_t thread_event(hipStream_t stream) {
    constexpr int kMaxDev = 64;
    thread_local hipEvent_t ev[kMaxDev] = {};
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    if (!ev[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&ev[dev], hipEventDisableTiming) != hipSuccess) ev[dev] = nullptr;
        if (cur != dev) (void)hipSetDevice(cur);
    }
    return ev[dev];
}

hipError_t radix_pass(uint64_t* const codes[2], uint32_t* const idx[2], int cur, int64_t N, int shift,
                      bool hist_ready, uint32_t* hist, uint32_t* totals, int64_t nblk,
                      const PackPart* ppart, BuildFlags* hflags, hipEvent_t ev, hipStream_t stream) {
    if (!hist_ready) {
        k_radix_hist<<<dim3((unsigned)nblk), dim3(kSortThreads), 0, stream>>>(codes[cur], N, shift, hist, nblk);
        SPC_TRY(hipGetLastError());
    }
    k_radix_rowscan<<<dim3(kRadix), dim3(256), 0, stream>>>(hist, nblk, totals, ppart, hflags);
    SPC_TRY(hipGetLastError());
    if (ev) SPC_TRY(hipEventRecord(ev, stream));
    k_radix_scatter<<<dim3((unsigned)nblk), dim3(kSortThreads), 0, stream>>>(
        codes[cur], idx[cur], N, shift, hist, nblk, totals, codes[cur ^ 1], idx[cur ^ 1]);
    return hipGetLastError();
}

// The distinct rows of each tile, then the
// map's totals (valid pairs, duplicates, the largest distinct-row count).
hipError_t finish(const ArenaLayout& al, char* arena, int64_t N, int K, const CountPart* cpart,
                  BuildFlags* hflags, hipStream_t stream) {
    uint32_t* dcount = (uint32_t*)(arena + al.dcount_off);
    if (N > 0) {
        k_tile_distinct<<<dim3((unsigned)(al.ntiles * kDistinctPerTile)), dim3(kDistinctRows), 0, stream>>>(
            (const int32_t*)(arena + al.nbr_off), N, al.Npad, K, dcount, (int32_t*)(arena + al.drow_off),
            (uint16_t*)(arena + al.smap_off));
        SPC_TRY(hipGetLastError());
    }
    k_finish<<<dim3(1), dim3(kFinishThreads), 0, stream>>>((const unsigned long long*)(arena + al.pairs_off),
                                                           dcount, N > 0 ? al.ntiles : 0,
                                                           N > 0 ? al.ntiles * kDistinctPerTile : 0, cpart,
                                                           (MapInfo*)(arena + al.info_off), hflags);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build(const int32_t* coords, int batches, int64_t N, int K, int dilation, int side,
                        const ArenaLayout& al, char* arena, const WorkspaceLayout& wl, char* ws,
                        hipStream_t stream, BuildFlags* host_flags) {
    uint64_t* const codes[2] = {(uint64_t*)(ws + wl.codes0), (uint64_t*)(ws + wl.codes1)};
    uint32_t* const idx[2] = {(uint32_t*)(ws + wl.idx0), (uint32_t*)(ws + wl.idx1)};
    uint32_t* hist = (uint32_t*)(ws + wl.hist);
    uint32_t* totals = (uint32_t*)(ws + wl.totals);
    PackPart* ppart = (PackPart*)(ws + wl.pack_part);
    CountPart* cpart = (CountPart*)(ws + wl.count_part);
    BrickSlot* table = (BrickSlot*)(ws + wl.table);
    BuildFlags* flags = (BuildFlags*)(ws + wl.flags);
    BuildFlags* hf_dev = nullptr;
    volatile BuildFlags* hf = host_flags_buffer(&hf_dev);
    if (!hf) return hipErrorOutOfMemory;
    const hipEvent_t ev = thread_event(stream);
    if (!ev) return hipErrorInvalidResourceHandle;
    const int64_t nblk = wl.nsort_blocks;

    CoordForm form;
    form.stride = batches > 0 ? 4 : 3;
    form.B = batches;
    form.log2S = 21 - batch_slab_log2(batches);
    form.margin = dilation * ((side - 1) / 2);
    k_pack<<<dim3((unsigned)nblk), dim3(kSortThreads), 0, stream>>>(coords, form, N, codes[0], idx[0], hist, nblk,
                                                                    ppart);
    SPC_TRY(hipGetLastError());
    // The first pass is needed whenever any bit varies.  Its scan kernel also
    // publishes the flags; the scatter is enqueued before the host waits for
    // them, so that the GPU sorts while the host reads how many passes remain.
    SPC_TRY(radix_pass(codes, idx, 0, N, 0, true, hist, totals, nblk, ppart, hf_dev, ev, stream));
    SPC_TRY(hipEventSynchronize(ev));
    if (hf->range_error) {
        host_flags->range_error = 1;
        return hipStreamSynchronize(stream);
    }

    // sort on the bits that differ across the set; higher bits are common
    const uint64_t x = hf->morton_xor_or;
    int bits = 0;
    while (bits < 64 && (x >> bits)) ++bits;
    const int passes = (bits + kRadixBits - 1) / kRadixBits;
    int cur = 1;
    for (int p = 1; p < passes; ++p) {
        SPC_TRY(radix_pass(codes, idx, cur, N, p * kRadixBits, false, hist, totals, nblk, nullptr, nullptr,
                           nullptr, stream));
        cur ^= 1;
    }

    k_brick_count<<<dim3(kCountBlocks), dim3(256), 0, stream>>>(codes[cur], N, cpart);
    SPC_TRY(hipGetLastError());
    const unsigned gblocks = (unsigned)std::min<int64_t>((N + 255) / 256, 2048);
    k_brick_fill<<<dim3(gblocks), dim3(256), 0, stream>>>(table, wl.log2_cap, cpart, flags);
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
    qa.tile_pairs = (unsigned long long*)(arena + al.pairs_off);
    SPC_TRY(run_tile_query(qa, al, stream));
    // the duplicate flag and the valid-pair count arrive in the host flags
    SPC_TRY(finish(al, arena, N, K, cpart, hf_dev, stream));
    SPC_TRY(hipStreamSynchronize(stream));
    host_flags->duplicate = hf->duplicate;
    host_flags->valid_pairs = hf->valid_pairs;
    host_flags->max_distinct = hf->max_distinct;
    return hipSuccess;
}

hipError_t launch_wrap(const int32_t* nbr, int64_t N, int K, const ArenaLayout& al, char* arena,
                       hipStream_t stream) {
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
    qa.tile_pairs = (unsigned long long*)(arena + al.pairs_off);
    SPC_TRY(run_tile_query(qa, al, stream));
    return finish(al, arena, N, K, nullptr, nullptr, stream);
}

hipError_t launch_export(const int32_t* nbr_m, const int32_t* order, int64_t N, int64_t Npad, int K,
                         int32_t* nbr_out, int32_t* order_out, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)(nbr_out ? K : 1));
    k_export<<<grid, dim3(256), 0, stream>>>(nbr_m, order, N, Npad, nbr_out, order_out);
    return hipGetLastError();
}

}  // namespace spc
