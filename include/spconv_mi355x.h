/*
 * spconv_mi355x.h -- C interface of libspconv_mi355x.so: the fused
 * gather-GEMM-accumulate of a submanifold sparse 3D convolution on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "mlx_backend/sparse_conv_metal.py": module docstring,
 * the kernel body and the `sparse_conv_metal` wrapper docstring):
 *
 *     out[n, co] = bias[co] + sum_k sum_ci feats[nbr[k, n], ci] * w[k, ci, co]
 *
 * nbr is a (K, N) int32 neighbour map, element k*N + n, whose value N marks a
 * missing neighbour (the page's pad row; it contributes nothing).  The (K, N, Ci)
 * gather is never materialised: one kernel accumulates straight from feats and w.
 *
 * Conventions shared by every call:
 *  - Pointers marked (dev) are HIP device memory owned by the caller; the
 *    library never allocates, frees or retains device memory.  Pointers marked
 *    (host) are ordinary host memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls enqueue work on it and return without waiting, except where noted.
 *  - Every call returns an int status (SPCONV_OK = 0, negative on error).
 *    Argument checks happen on the host before any launch; a failed check
 *    enqueues nothing.  spconv_last_error() gives a text for the last failure
 *    of the calling thread.
 *  - Device buffers must be 256-byte aligned (arena, workspace) or 16-byte
 *    aligned (coords, feats, w, out, nbr); torch allocations satisfy both.
 */
#ifndef SPCONV_MI355X_H
#define SPCONV_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPCONV_ABI_VERSION 1

enum spconv_status {
    SPCONV_OK = 0,
    SPCONV_E_INVALID = -1,      /* bad argument: null pointer, bad K, bad alignment, ... */
    SPCONV_E_UNSUPPORTED = -2,  /* valid but not implemented (e.g. a channel count)      */
    SPCONV_E_COORD_RANGE = -3,  /* a coordinate outside [-2^20, 2^20)                    */
    SPCONV_E_DUPLICATE = -4,    /* two voxels share a coordinate                          */
    SPCONV_E_WORKSPACE = -5,    /* arena or workspace smaller than required               */
    SPCONV_E_HIP = -6           /* a HIP runtime call failed                              */
};

enum spconv_dtype {
    SPCONV_F32 = 0,             /* feats, w, out float32                                  */
    SPCONV_BF16 = 1             /* feats, w, out bfloat16; accumulation is fp32 either way */
};

/* Opaque host-side handle of a built neighbour map.  The map's device data
 * lives in the caller's arena, which must outlive every use of the handle. */
typedef struct spconv_nmap spconv_nmap;

int spconv_abi_version(void);

/* Byte sizes of the persistent arena (the map, its row schedule and block
 * masks: about (4K+4)*N bytes) and of the build-only workspace (sort buffers
 * and brick table: about 24N + 32*2^ceil(log2(2N)) bytes) for N voxels and K
 * offsets.  Host only, pure.  K must be >= 1. */
int spconv_nmap_sizes(int64_t N, int K, size_t* arena_bytes, size_t* workspace_bytes);

/* Build the neighbour map of N active voxels.
 *   coords   (dev) int32 (N, 3): x, y, z of voxel n at 3n..3n+2, each in
 *            [-2^20, 2^20), all distinct.  The caller's order defines n.
 *   K        an odd cube (1, 27, 125, ...): offsets o_k, k = ((a*s)+b)*s + c,
 *            s = cbrt(K), o_k = (a-r, b-r, c-r) * dilation, r = (s-1)/2
 *            (x slowest, z fastest; centre k = (K-1)/2).  The page leaves the
 *            offset numbering to the map's builder; this is the numbering of a
 *            dense 3D cross-correlation with padding r*dilation.
 *   dilation >= 1.
 *   nbr[k, n] = m if coords[m] == coords[n] + o_k, else N  (page: the
 *   `sparse_conv_metal` wrapper docstring gives the (K, N) int32 layout and
 *   the N sentinel).
 * The map is stored in the arena in an internal row order (Morton order of the
 * voxels, refined by sorting rows on their validity masks inside 128-row
 * half tiles); spconv_nmap_export returns it in the caller's order.
 * Waits on `stream` twice: mid-build for the coordinate range check and the
 * number of Morton bits that vary (which fixes the sort passes; the first sort
 * pass is already queued, so the GPU keeps working meanwhile), and at the end
 * (SPCONV_E_DUPLICATE, and the valid-pair count kept in the handle).  Both
 * results arrive in a small pinned host buffer that the kernels write
 * directly; the waits use one HIP event per device.  The buffer (128 bytes)
 * and the events belong to the calling thread and are kept until the process
 * ends: the library never frees them, since at process exit the HIP runtime
 * may already be gone.  The workspace may be reused or freed when this
 * returns.
 * On success *out receives a handle to release with spconv_nmap_destroy. */
int spconv_build_nmap(const int32_t* coords, int64_t N, int K, int dilation,
                      void* arena, size_t arena_bytes,
                      void* workspace, size_t workspace_bytes,
                      void* stream, spconv_nmap** out);

/* spconv_build_nmap for several scenes in one map (batched coordinates; the
 * pages' voxel sets carry no batch field, so this is the library's form):
 *   coords   (dev) int32 (N, 4): b, x, y, z of voxel n at 4n..4n+3, b in
 *            [0, batches); voxels are neighbours only within one batch.
 *   Each batch occupies its own slab of S = 2^21 / B' x-values, B' = batches
 *   rounded up to a power of two: its x must lie in [-S/2 + r*d, S/2 - r*d)
 *   (r*d = the stencil's reach), y and z in [-2^20, 2^20); otherwise
 *   SPCONV_E_COORD_RANGE.  Too many batches for the reach gives
 *   SPCONV_E_UNSUPPORTED.  Arena and workspace sizes, ordering, errors and
 *   synchronisation are those of spconv_build_nmap. */
int spconv_build_nmap_batched(const int32_t* coords, int64_t N, int batches, int K, int dilation,
                              void* arena, size_t arena_bytes,
                              void* workspace, size_t workspace_bytes,
                              void* stream, spconv_nmap** out);

/* Wrap a caller-made (K, N) int32 map (dev, element k*N + n) into a handle, as
 * the page's operator receives one.  Values outside [0, N) are treated as
 * missing.  Rows keep the caller's order apart from the in-tile mask sort.
 * Needs an arena of spconv_nmap_sizes(N, K) bytes, no workspace, no sync. */
int spconv_nmap_wrap(const int32_t* nbr, int64_t N, int K,
                     void* arena, size_t arena_bytes, void* stream, spconv_nmap** out);

/* Copy the map out in the caller's order.
 *   nbr_out   (dev) int32 (K, N), or NULL
 *   order_out (dev) int32 (N): row i of the internal schedule holds voxel
 *             order_out[i]; or NULL
 * Asynchronous on `stream`. */
int spconv_nmap_export(const spconv_nmap* h, int32_t* nbr_out, int32_t* order_out, void* stream);

/* Sizes of a handle; valid_pairs (the number of (k, n) entries != N) is read
 * from the device, which synchronises `stream` the first time.  Any output
 * pointer may be NULL. */
int spconv_nmap_info(const spconv_nmap* h, int64_t* N, int* K, int* dilation,
                     int64_t* valid_pairs, void* stream);

/* The fused forward (page: the kernel body and the wrapper).
 *   feats (dev) (N, Ci) row-major (N+1 rows are accepted; row N is never read)
 *   w     (dev) (K, Ci, Co) row-major, K = the handle's K
 *   bias  (dev) float32 (Co,), or NULL for zero
 *   out   (dev) (N, Co) row-major, written completely
 *   dtype SPCONV_F32 or SPCONV_BF16 for feats, w and out together.
 * Accumulation is fp32 over all K offsets; bias is added in fp32 and the sum
 * is rounded once (round-to-nearest-even) to the output type.  (The page adds
 * the bias after rounding the accumulator to the weight type; one rounding is
 * this library's choice.)
 * Supported: Ci in {32, 64, 128, 256}, Co a multiple of 32 up to 4096.
 * Others return SPCONV_E_UNSUPPORTED.  Asynchronous, no synchronisation:
 * two calls with the same inputs give bit-identical outputs.
 * bfloat16 with Ci = 128 and Co a multiple of 64 runs the kernel over each
 * tile's distinct neighbour rows, which reads w packed: this call packs w
 * into a stream-ordered allocation of K*Ci*Co*2 bytes (hipMallocAsync) that
 * it frees on `stream` after the forward; spconv_forward_packed with a
 * caller's pack gives the same bits without it.  That kernel's workgroups
 * take tiles from atomic counters (which workgroup computes a tile changes
 * from run to run, how it is computed does not) held in a library-owned
 * device array of 8192 counter slots per device: each launch takes Co/128
 * or Co/64 slots in turn and leaves them at zero when it completes, so
 * launches in flight at the same time share counters only if 8192 slots
 * were handed out between their starts.  N = 0 is a no-op. */
int spconv_forward(const void* feats, const spconv_nmap* nmap, const void* w,
                   const float* bias, void* out, int Ci, int Co, int dtype, void* stream);

/* The forward with feats in a dtype of their own (page: the wrapper casts
 * feats to the weights' dtype before the kernel runs).
 *   feats_dtype  SPCONV_F32 or SPCONV_BF16: the element type of feats
 *   dtype        the element type of w and out
 *   wpack        (dev) optional: spconv_pack_weights(w), used where the
 *                bfloat16 forward has a packed form; or NULL
 *   workspace    (dev) optional, 256-byte aligned, of at least
 *                spconv_forward_mixed_workspace_size bytes; or NULL
 * float32 -> bfloat16 rounds to nearest even (NaN stays NaN); bfloat16 ->
 * float32 is exact.  Without a workspace each gathered value is converted as
 * it is loaded.  With one (float32 feats into bfloat16 weights only; the size
 * is 0 for the other pairings and the argument is then ignored), a streaming
 * pass first writes the cast features into it and the bfloat16 forward runs
 * on them: the page's order, and faster at Ci = 128 and 256.  Both give the
 * forward of the cast features up to accumulation order.  With feats_dtype ==
 * dtype this is spconv_forward (same kernels).  Other arguments, limits,
 * errors and ordering are spconv_forward's.  Only the work this call
 * enqueues on `stream` writes and reads the workspace; it may be reused once
 * that work is done. */
int spconv_forward_mixed_workspace_size(int64_t N, int Ci, int feats_dtype, int dtype, size_t* bytes);
int spconv_forward_mixed(const void* feats, int feats_dtype, const spconv_nmap* nmap, const void* w,
                         const void* wpack, const float* bias, void* out, int Ci, int Co, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Packed weights: an optional second copy of w (the same size) in the order
 * the bf16 forward reads it, so that the kernel loads each offset's slice with
 * plain 16-byte accesses instead of transposing w again for every tile.
 *   Ci = 128, Co a multiple of 64: fragment order.  16-byte unit
 *     e = (((k (Co/64) + c) 4 + s) 4 + j) 64 + l, lane l = m + 16 q, holds
 *     w[k][32 s + 8 q .. 32 s + 8 q + 7][64 c + 16 (m >> 2) + 4 j + (m & 3)]:
 *     lane l's matrix-core operand of output tile j, input-channel step s.
 *   Ci = 256, or Ci = 128 with other Co: per offset k and tile of BN output
 *     channels, 8 input channels x one output channel per 16-byte unit, output
 *     channels in the order the matrix-core tiles use.
 * The page's operator takes w as is; packing is this library's own
 * acceleration and is computed from w alone.
 *
 * spconv_pack_weights_size: bytes of the packed copy for (K, Ci, Co, dtype);
 * 0 when the forward has no packed form for that configuration (float32, or
 * Ci < 128).  Host only.
 * spconv_pack_weights: writes the packed copy of w (dev, (K, Ci, Co)
 * row-major) into wpack (dev, 16-byte aligned, at least the size above);
 * asynchronous on `stream`; a no-op when the size is 0.  wpack must be
 * repacked whenever w changes. */
int spconv_pack_weights_size(int K, int Ci, int Co, int dtype, size_t* bytes);
int spconv_pack_weights(const void* w, int K, int Ci, int Co, int dtype,
                        void* wpack, size_t wpack_bytes, void* stream);

/* spconv_forward with packed weights: the same operation, arguments and
 * result (bit for bit) as spconv_forward, plus wpack packed from the same w
 * for the handle's K; no allocation.  w is still required: configurations the
 * packed kernels do not serve (Ci = 256 feats of 4 GiB or more) read it
 * directly.  wpack may be NULL only when spconv_pack_weights_size gives 0. */
int spconv_forward_packed(const void* feats, const spconv_nmap* nmap, const void* w,
                          const void* wpack, const float* bias, void* out,
                          int Ci, int Co, int dtype, void* stream);

/* Input gradient of spconv_forward (the adjoint of its linear map in feats;
 * the page gives the forward formula, module docstring of
 * "mlx_backend/sparse_conv_metal.py", and the gradient follows from it):
 *   dfeats[m, ci] = sum over (k, n) with nbr[k, n] == m of
 *                   sum_co dout[n, co] * w[k, ci, co]
 *   dout     (dev) (N, Co), dtype as w;  w (dev) (K, Ci, Co)
 *   dfeats   (dev) (N, Ci) written, dtype as w; no bias term
 *   workspace (dev) spconv_dgrad_workspace_size bytes, 256-byte aligned,
 *            caller-owned, free after the call's work has run
 * The map must come from spconv_build_nmap: a map of a symmetric stencil is
 * its own mirror, nbr[K-1-k, nbr[k, n]] = n, so the gradient is the forward
 * over dout with the weights w'[k] = w[K-1-k]^T, which this call writes into
 * the workspace (and packs there when the bf16 kernel has a packed form)
 * before running the forward kernels with Ci and Co exchanged.  A wrapped map
 * gives SPCONV_E_UNSUPPORTED; so does a (Ci, Co) for which the exchanged
 * forward has no kernel (Co in {32, 64, 128, 256}, Ci a multiple of 32 up to
 * 4096).  Asynchronous on `stream`, no allocation, no synchronisation. */
int spconv_dgrad_workspace_size(int K, int Ci, int Co, int dtype, size_t* bytes);
int spconv_dgrad(const void* dout, const spconv_nmap* nmap, const void* w,
                 void* workspace, size_t workspace_bytes, void* dfeats,
                 int Ci, int Co, int dtype, void* stream);

/* spconv_dgrad without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same operation, arguments, result and errors as
 * spconv_dgrad; the mirrored and packed weights go into a fixed scratch array
 * of SPCONV_NOALLOC_SCRATCH_BYTES inside the library (one per device, taken
 * at the first call on that device and held until the process ends).
 * Configurations whose spconv_dgrad_workspace_size exceeds it return
 * SPCONV_E_WORKSPACE (K = 27 fits every supported Ci, Co <= 256 in either
 * dtype).  The call allocates nothing.  Every call on one device shares that
 * device's scratch: calls that overlap in time on one device (concurrent
 * streams, other host threads) race and must be serialised by the caller;
 * calls in order on one stream are safe.  Nothing in the scratch needs to
 * start at zero: each call writes all of the part it reads. */
#define SPCONV_NOALLOC_SCRATCH_BYTES (16u << 20)
int spconv_dgrad_noalloc(const void* dout, const spconv_nmap* nmap, const void* w, void* dfeats,
                         int Ci, int Co, int dtype, void* stream);

/* Weight gradient of spconv_forward (its derivative with respect to w,
 * contracted with dout; the page gives the forward formula, module docstring
 * of "mlx_backend/sparse_conv_metal.py"):
 *   dw[k, ci, co] = sum over n with nbr[k, n] present of feats[nbr[k, n], ci] * dout[n, co]
 *   feats    (dev) (N or N+1, Ci) and dout (dev) (N, Co), one dtype
 *   dw       (dev) (K, Ci, Co) written in that dtype (fp32 sums, one rounding)
 *   workspace (dev) spconv_wgrad_workspace_size bytes, 256-byte aligned,
 *            caller-owned: fp32 partial sums of row chunks (a few times
 *            K*Ci*Co*4 bytes), added up in a fixed order, so the result is
 *            deterministic
 * Ci and Co: multiples of 32 up to 4096.  Works with built and wrapped maps.
 * Asynchronous on `stream`, no allocation, no synchronisation, no atomics. */
int spconv_wgrad_workspace_size(int64_t N, int K, int Ci, int Co, int dtype, size_t* bytes);
int spconv_wgrad(const void* feats, const void* dout, const spconv_nmap* nmap,
                 void* workspace, size_t workspace_bytes, void* dw,
                 int Ci, int Co, int dtype, void* stream);

/* Release a handle (host memory only; the arena stays the caller's). */
void spconv_nmap_destroy(spconv_nmap* h);

const char* spconv_status_string(int status);
const char* spconv_last_error(void);
/* The same thread-local text under the name the hot-path boundary proposes
 * for SPCONV_E_HIP failures (it covers every failure, HIP or not). */
const char* spconv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPCONV_MI355X_H */
