// Internal declarations shared by the HIP sources of libspconv_mi355x.
// Not installed; the public interface is include/spconv_mi355x.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spconv_mi355x.h"

namespace spc {

// Rows of the locality schedule are grouped in tiles of this many rows.  The
// builder sorts rows by validity mask inside each half tile (kSortRows rows)
// and records, per (tile, offset), which 16-row blocks hold at least one
// present neighbour.
constexpr int kTileRows = 256;
constexpr int kSortRows = 128;
constexpr int kBlockRows = 16;
constexpr int kBlocksPerTile = kTileRows / kBlockRows;  // 16 -> one uint16 per (tile, k)

// Workgroup barrier without the memory fence of __syncthreads, which makes
// each wave first wait for all of its outstanding loads, DMAs and stores.
// Kernels that keep loads in flight across a barrier use this and issue the
// waits the barrier needs themselves.  The clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kCoordBias = 1 << 20;                      // coords in [-2^20, 2^20)
constexpr uint64_t kEmptyKey = ~0ull;

constexpr int kSortThreads = 1024;                        // 16 waves: four per SIMD
constexpr int kSortItems = 4;
constexpr int kSortChunk = kSortThreads * kSortItems;    // elements per sort block
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;

// Device-side status of a build, read back by the host (one 128-byte line).
// Every field is written unconditionally by the kernel that owns it, so the
// header needs no clearing between builds.  Totals over many workgroups are
// formed from per-workgroup partials by one small kernel: device-scope atomics
// on one address from thousands of workgroups serialise in the memory system.
struct BuildFlags {
    unsigned long long morton_xor_or;   // OR over voxels of (code ^ code of voxel 0)
    unsigned long long valid_pairs;     // present (row, offset) pairs of the map
    uint32_t range_error;               // a coordinate outside [-2^20, 2^20)
    uint32_t duplicate;                 // two voxels with the same coordinate
    uint32_t nbricks;                   // occupied 4x4x4 bricks
    uint32_t log2_bricks;               // log2 of the brick table's capacity in use
    uint32_t max_distinct;              // most distinct neighbour rows of a tile (kNoDistinct: over the cap)
    uint32_t pad0;
    uint64_t pad[11];
};

// Per-workgroup partials of the pack and brick-count kernels.
struct PackPart {
    unsigned long long xor_or;
    uint32_t bad;
    uint32_t pad;
};
struct CountPart {
    uint32_t heads;
    uint32_t dup;
};
constexpr int kCountBlocks = 256;   // workgroups of the brick count

// Persistent per-map device header (lives in the arena).
struct MapInfo {
    unsigned long long valid_pairs;
    uint32_t max_distinct;
    uint32_t pad0;
    uint64_t pad[30];
};

// Distinct neighbour rows of a half tile (kDistinctRows = kSortRows rows of
// the schedule): the rows that some row of it has as present neighbours, for
// maps of at most kDistinctMaxK offsets, staged by the forward in LDS, which
// holds kDistinctCap rows.  Most half tiles need one staging pass: all their
// distinct rows are listed (count n <= kDistinctCap, dcount = n).  A half
// tile with more, in a 27-offset map, is staged in three passes, one per
// layer of nine offsets (9p .. 9p + 8, the map's x offset), each with its own
// list of at most kDistinctCap rows at entry kDistinctCap p (dcount =
// kLayerPasses | n0 | n1 << 10 | n2 << 20); a row needed by two layers is
// listed in both.  Otherwise dcount = kNoDistinct and there are no lists.
// slot_map[half][k][slot_pos(r)] (uint16, row r of the half tile; the 8 codes
// of row n of the 8 blocks contiguous) encodes the slot s, in the list of
// offset k's pass, of that row's neighbour at offset k as (s << 4) | 2 ((s >>
// 1) & 7): the 16-byte unit index of the row's first chunk in the forward's
// LDS row stage and the XOR swizzle of its chunks.  A missing neighbour has
// slot kDistinctCap (the stage's zero row).
constexpr int kDistinctRows = kSortRows;
constexpr int kDistinctPerTile = kTileRows / kDistinctRows;
constexpr int kDistinctCap = 315;
constexpr int kDistinctLayers = 3;
constexpr int kDistinctListCap = kDistinctLayers * kDistinctCap;
constexpr int kDistinctMaxK = 27;
constexpr uint32_t kLayerPasses = 0x80000000u;
static_assert(kDistinctCap < 1024, "three counts in one word");
__host__ __device__ constexpr uint32_t slot_code(uint32_t s) { return (s << 4) | (2u * ((s >> 1) & 7u)); }
__host__ __device__ constexpr int layer_rows(uint32_t dcount, int p) { return (int)((dcount >> (10 * p)) & 1023u); }
// position of row r (block b = r >> 4, row n = r & 15 of it) in a slot map
__host__ __device__ constexpr int slot_pos(int r) { return (r & 15) * (kDistinctRows / 16) + (r >> 4); }
constexpr uint32_t kNoDistinct = 0xFFFFFFFFu;

// Open-addressing hash slot of one occupied 4x4x4 brick: its key (the
// Morton code of the brick), the first position of its voxels in the Morton
// order, and a 64-bit mask of which of its 64 cells are occupied (cell =
// the low 6 Morton bits).  The brick's voxels are consecutive in the order.
struct alignas(32) BrickSlot {
    unsigned long long key;
    uint32_t start;
    uint32_t pad0;
    unsigned long long mask;
    unsigned long long pad1;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Arena / workspace layouts (byte offsets), computed identically by the size
// query and by the builder.
struct ArenaLayout {
    int64_t Npad;
    int64_t ntiles;
    size_t nbr_off, order_off, mask_off, pairs_off, info_off;
    size_t dcount_off, drow_off, smap_off, total;
};

struct WorkspaceLayout {
    int64_t nsort_blocks;
    int log2_cap;
    size_t codes0, codes1, idx0, idx1, hist, totals, pack_part, count_part, table, flags, total;
};

ArenaLayout arena_layout(int64_t N, int K);
WorkspaceLayout workspace_layout(int64_t N);

// Odd cube side of K, or -1.
int cube_side(int K);
// log2 of the number of x-slabs that batched coordinates use (batches rounded
// up to a power of two; 0 for unbatched or one batch).
int batch_slab_log2(int batches);

// Launchers (host).  Return hipError_t of the launches.
// batches = 0: coords (N, 3) x, y, z; batches >= 1: coords (N, 4) b, x, y, z.
hipError_t launch_build(const int32_t* coords, int batches, int64_t N, int K, int dilation, int side,
                        const ArenaLayout& al, char* arena, const WorkspaceLayout& wl, char* ws,
                        hipStream_t stream, BuildFlags* host_flags);
hipError_t launch_wrap(const int32_t* nbr, int64_t N, int K, const ArenaLayout& al, char* arena,
                       hipStream_t stream);
hipError_t launch_export(const int32_t* nbr_m, const int32_t* order, int64_t N, int64_t Npad, int K,
                         int32_t* nbr_out, int32_t* order_out, hipStream_t stream);

struct ForwardArgs {
    const void* feats;
    const int32_t* nbr_m;
    const int32_t* order;
    const uint16_t* blkmask;
    const uint32_t* dcount;     // distinct rows per half tile (kNoDistinct: over the cap)
    const int32_t* drow;        // [half tile][kDistinctListCap] caller indices of the distinct rows
    const uint16_t* smap;       // [half tile][K][16][8] slot codes
    int64_t max_distinct;       // most distinct rows of any half tile; -1 when not known on the host
    const void* w;
    const void* wpack;    // packed weights (spconv_pack_weights), or NULL
    const float* bias;
    void* out;
    int64_t N, Npad;
    int K, Ci, Co, dtype;
    int feats_dtype;      // dtype of feats; cast to `dtype` (w's) as it is gathered
    void* cast_ws;        // fp32 feats, bf16 w: cast into this (cast_workspace_bytes) first, or NULL
};
// Workspace for the separate cast pass of the mixed forward (0: no such pass).
size_t cast_workspace_bytes(int64_t N, int Ci, int feats_dtype, int dtype);
// Returns hipErrorInvalidValue when (dtype, Ci, Co) has no kernel.
hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream);
bool forward_supported(int dtype, int Ci, int Co);
// Whether (dtype, feature dtype, Ci, Co) runs the tile kernel over each tile's
// distinct rows, which takes the weights in their packed form only.
bool tile_forward(int dtype, int feats_dtype, int Ci, int Co);
// Bytes of the packed weights for (K, Ci, Co, dtype); 0 when the forward has
// no packed form for this configuration (the pack is then empty).
size_t packed_weight_bytes(int K, int Ci, int Co, int dtype);
hipError_t launch_pack_weights(const void* w, int K, int Ci, int Co, int dtype, void* wpack, hipStream_t stream);
// wt[k][co][ci] = w[K-1-k][ci][co] (the input gradient's weights).
hipError_t launch_mirror_weights(const void* w, int K, int Ci, int Co, int dtype, void* wt, hipStream_t stream);

struct WgradArgs {
    const void* feats;
    const void* dout;
    const int32_t* nbr_m;
    const int32_t* order;
    const uint16_t* blkmask;
    const uint32_t* dcount;   // the map's distinct-row lists (see above)
    const int32_t* drow;
    const uint16_t* smap;
    int64_t max_distinct;     // -1: unknown; > kDistinctListCap: some half tile has no lists
    void* workspace;          // wgrad_workspace_bytes: fp32 partials per row chunk
    void* dw;
    int64_t N, Npad;
    int K, Ci, Co, dtype;
};
bool wgrad_supported(int dtype, int Ci, int Co);
size_t wgrad_workspace_bytes(int64_t N, int K, int Ci, int Co, int dtype);
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t stream);

}  // namespace spc

// Opaque handle of the public interface.
struct spconv_nmap {
    uint32_t magic;
    int64_t N, Npad, ntiles;
    int K, dilation;
    int wrapped;
    int32_t* nbr_m;     // [K][Npad] caller indices, schedule row order, sentinel N
    int32_t* order;     // [Npad]   schedule row -> caller index (-1 for padding rows)
    uint16_t* blkmask;  // [ntiles][K] bit b: some row of 16-row block b is present
    uint32_t* dcount;   // [2 ntiles] distinct neighbour rows of each half tile
    int32_t* drow;      // [2 ntiles][kDistinctListCap] their caller indices
    uint16_t* smap;     // [2 ntiles][K][16][8] slot of each (row, offset)'s neighbour
    spc::MapInfo* info;
    int64_t valid_pairs;  // host copy, -1 until read
    int64_t max_distinct; // host copy, -1 until known
};
constexpr uint32_t kNmapMagic = 0x53504e4du;
