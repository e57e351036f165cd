// C interface of libspconv_mi355x: argument checks, handle management and
// dispatch to the builder and forward launchers.  Every check runs on the host
// before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "spconv_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(SPCONV_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The sentinel N has to fit the int32 map (the page's kernel compares
// int nbr >= (int)N).
constexpr int64_t kMaxN = (int64_t)INT32_MAX - 1;
constexpr int kMaxKApi = 1000;

int check_nk(int64_t N, int K) {
    if (N < 0) return fail(SPCONV_E_INVALID, "N must be >= 0 (got %lld)", (long long)N);
    if (N > kMaxN) return fail(SPCONV_E_UNSUPPORTED, "N must be < 2^31-1 (got %lld)", (long long)N);
    if (K < 1 || K > kMaxKApi) return fail(SPCONV_E_INVALID, "K must be in [1, %d] (got %d)", kMaxKApi, K);
    return SPCONV_OK;
}

spconv_nmap* make_handle(int64_t N, int K, int dilation, int wrapped, const spc::ArenaLayout& al,
                         char* arena) {
    spconv_nmap* h = new (std::nothrow) spconv_nmap;
    if (!h) return nullptr;
    h->magic = kNmapMagic;
    h->N = N;
    h->Npad = al.Npad;
    h->ntiles = al.ntiles;
    h->K = K;
    h->dilation = dilation;
    h->wrapped = wrapped;
    h->nbr_m = (int32_t*)(arena + al.nbr_off);
    h->order = (int32_t*)(arena + al.order_off);
    h->blkmask = (uint16_t*)(arena + al.mask_off);
    h->dcount = (uint32_t*)(arena + al.dcount_off);
    h->drow = (int32_t*)(arena + al.drow_off);
    h->smap = (uint16_t*)(arena + al.smap_off);
    h->info = (spc::MapInfo*)(arena + al.info_off);
    h->valid_pairs = (N == 0) ? 0 : -1;
    h->max_distinct = (N == 0) ? 0 : -1;
    return h;
}

bool valid_handle(const spconv_nmap* h) { return h && h->magic == kNmapMagic; }

// Scratch of spconv_dgrad_noalloc: the input gradient's mirrored weights and
// their packed form, for callers that cannot allocate.  Each device holds its
// own copy from the library's first use there until the process ends.  In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = SPCONV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream).
int scratch_address(void* stream, void** ptr, const char* where) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, where);
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(SPCONV_E_UNSUPPORTED, "%s: device %d beyond the %d this library serves", where, dev,
                    kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_fail(e, where);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, where);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_fail(e, where);
        if (!p || !aligned(p, 256)) return fail(SPCONV_E_HIP, "%s: scratch address %p not usable", where, p);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SPCONV_OK;
}

}  // namespace

extern "C" {

int spconv_abi_version(void) { return SPCONV_ABI_VERSION; }

const char* spconv_last_error(void) { return g_last_error; }
const char* spconv_last_hip_error(void) { return g_last_error; }

const char* spconv_status_string(int status) {
    switch (status) {
        case SPCONV_OK: return "ok";
        case SPCONV_E_INVALID: return "invalid argument";
        case SPCONV_E_UNSUPPORTED: return "unsupported configuration";
        case SPCONV_E_COORD_RANGE: return "coordinate out of range [-2^20, 2^20)";
        case SPCONV_E_DUPLICATE: return "duplicate coordinate";
        case SPCONV_E_WORKSPACE: return "arena or workspace too small";
        case SPCONV_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int spconv_nmap_sizes(int64_t N, int K, size_t* arena_bytes, size_t* workspace_bytes) {
    int rc = check_nk(N, K);
    if (rc) return rc;
    if (arena_bytes) *arena_bytes = spc::arena_layout(N, K).total;
    if (workspace_bytes) *workspace_bytes = spc::workspace_layout(N).total;
    return SPCONV_OK;
}

static int build_impl(const int32_t* coords, int batches, int64_t N, int K, int dilation, void* arena,
                      size_t arena_bytes, void* workspace, size_t workspace_bytes, void* stream,
                      spconv_nmap** out, const char* name) {
    if (!out) return fail(SPCONV_E_INVALID, "out handle pointer is NULL");
    *out = nullptr;
    int rc = check_nk(N, K);
    if (rc) return rc;
    const int side = spc::cube_side(K);
    if (side < 0) return fail(SPCONV_E_INVALID, "K must be an odd cube 1, 27, 125, ... (got %d)", K);
    if (dilation < 1) return fail(SPCONV_E_INVALID, "dilation must be >= 1 (got %d)", dilation);
    if ((int64_t)dilation * (side - 1) / 2 >= (1 << 20))
        return fail(SPCONV_E_UNSUPPORTED, "dilation * radius must be < 2^20");
    if (batches > 0) {
        if (batches > (1 << 20)) return fail(SPCONV_E_UNSUPPORTED, "at most 2^20 batches (got %d)", batches);
        // each batch's x-slab must be wider than twice the stencil's reach
        const int64_t half = (int64_t)1 << (20 - spc::batch_slab_log2(batches));
        if ((int64_t)dilation * (side - 1) / 2 >= half)
            return fail(SPCONV_E_UNSUPPORTED, "%d batches leave x-slabs of %lld values, too narrow for "
                                              "dilation %d and K=%d", batches, (long long)(2 * half), dilation, K);
    }
    const spc::ArenaLayout al = spc::arena_layout(N, K);
    const spc::WorkspaceLayout wl = spc::workspace_layout(N);
    if (!arena) return fail(SPCONV_E_INVALID, "arena is NULL");
    if (!aligned(arena, 256)) return fail(SPCONV_E_INVALID, "arena must be 256-byte aligned");
    if (arena_bytes < al.total)
        return fail(SPCONV_E_WORKSPACE, "arena has %zu bytes, needs %zu", arena_bytes, al.total);
    if (N > 0) {
        if (!coords) return fail(SPCONV_E_INVALID, "coords is NULL");
        if (!aligned(coords, 4)) return fail(SPCONV_E_INVALID, "coords must be 4-byte aligned");
        if (!workspace) return fail(SPCONV_E_INVALID, "workspace is NULL");
        if (!aligned(workspace, 256)) return fail(SPCONV_E_INVALID, "workspace must be 256-byte aligned");
        if (workspace_bytes < wl.total)
            return fail(SPCONV_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                        wl.total);
    }
    spconv_nmap* h = make_handle(N, K, dilation, 0, al, (char*)arena);
    if (!h) return fail(SPCONV_E_INVALID, "out of host memory");
    if (N == 0) {
        *out = h;
        return SPCONV_OK;
    }
    spc::BuildFlags flags;
    memset(&flags, 0, sizeof flags);
    hipError_t e = spc::launch_build(coords, batches, N, K, dilation, side, al, (char*)arena, wl,
                                     (char*)workspace, (hipStream_t)stream, &flags);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, name);
    }
    if (flags.range_error) {
        delete h;
        if (batches > 0) {
            const int64_t half = (int64_t)1 << (20 - spc::batch_slab_log2(batches));
            const int64_t reach = (int64_t)dilation * (side - 1) / 2;
            return fail(SPCONV_E_COORD_RANGE,
                        "a batch index outside [0, %d), an x outside [%lld, %lld) or a y, z outside [-2^20, 2^20)",
                        batches, (long long)(-half + reach), (long long)(half - reach));
        }
        return fail(SPCONV_E_COORD_RANGE, "a coordinate lies outside [-2^20, 2^20)");
    }
    if (flags.duplicate) {
        delete h;
        return fail(SPCONV_E_DUPLICATE, "two voxels share a coordinate");
    }
    h->valid_pairs = (int64_t)flags.valid_pairs;
    h->max_distinct = flags.max_distinct == spc::kNoDistinct ? (int64_t)spc::kDistinctListCap + 1
                                                              : (int64_t)flags.max_distinct;
    *out = h;
    return SPCONV_OK;
}

int spconv_build_nmap(const int32_t* coords, int64_t N, int K, int dilation, void* arena,
                      size_t arena_bytes, void* workspace, size_t workspace_bytes, void* stream,
                      spconv_nmap** out) {
    return build_impl(coords, 0, N, K, dilation, arena, arena_bytes, workspace, workspace_bytes, stream, out,
                      "spconv_build_nmap");
}

int spconv_build_nmap_batched(const int32_t* coords, int64_t N, int batches, int K, int dilation, void* arena,
                              size_t arena_bytes, void* workspace, size_t workspace_bytes, void* stream,
                              spconv_nmap** out) {
    if (batches < 1) return fail(SPCONV_E_INVALID, "batches must be >= 1 (got %d)", batches);
    return build_impl(coords, batches, N, K, dilation, arena, arena_bytes, workspace, workspace_bytes, stream,
                      out, "spconv_build_nmap_batched");
}

int spconv_nmap_wrap(const int32_t* nbr, int64_t N, int K, void* arena, size_t arena_bytes,
                     void* stream, spconv_nmap** out) {
    if (!out) return fail(SPCONV_E_INVALID, "out handle pointer is NULL");
    *out = nullptr;
    int rc = check_nk(N, K);
    if (rc) return rc;
    const spc::ArenaLayout al = spc::arena_layout(N, K);
    if (!arena) return fail(SPCONV_E_INVALID, "arena is NULL");
    if (!aligned(arena, 256)) return fail(SPCONV_E_INVALID, "arena must be 256-byte aligned");
    if (arena_bytes < al.total)
        return fail(SPCONV_E_WORKSPACE, "arena has %zu bytes, needs %zu", arena_bytes, al.total);
    if (N > 0 && !nbr) return fail(SPCONV_E_INVALID, "nbr is NULL");
    if (N > 0 && !aligned(nbr, 4)) return fail(SPCONV_E_INVALID, "nbr must be 4-byte aligned");
    spconv_nmap* h = make_handle(N, K, 1, 1, al, (char*)arena);
    if (!h) return fail(SPCONV_E_INVALID, "out of host memory");
    if (N > 0) {
        hipError_t e = spc::launch_wrap(nbr, N, K, al, (char*)arena, (hipStream_t)stream);
        if (e != hipSuccess) {
            delete h;
            return hip_fail(e, "spconv_nmap_wrap");
        }
    }
    *out = h;
    return SPCONV_OK;
}

int spconv_nmap_export(const spconv_nmap* h, int32_t* nbr_out, int32_t* order_out, void* stream) {
    if (!valid_handle(h)) return fail(SPCONV_E_INVALID, "invalid handle");
    if ((nbr_out && !aligned(nbr_out, 4)) || (order_out && !aligned(order_out, 4)))
        return fail(SPCONV_E_INVALID, "outputs must be 4-byte aligned");
    if (h->N == 0 || (!nbr_out && !order_out)) return SPCONV_OK;
    hipError_t e = spc::launch_export(h->nbr_m, h->order, h->N, h->Npad, h->K, nbr_out, order_out,
                                      (hipStream_t)stream);
    return e == hipSuccess ? SPCONV_OK : hip_fail(e, "spconv_nmap_export");
}

int spconv_nmap_info(const spconv_nmap* h, int64_t* N, int* K, int* dilation, int64_t* valid_pairs,
                     void* stream) {
    if (!valid_handle(h)) return fail(SPCONV_E_INVALID, "invalid handle");
    if (N) *N = h->N;
    if (K) *K = h->K;
    if (dilation) *dilation = h->dilation;
    if (valid_pairs) {
        if (h->valid_pairs < 0) {
            unsigned long long v = 0;
            hipError_t e = hipMemcpyAsync(&v, &h->info->valid_pairs, sizeof v, hipMemcpyDeviceToHost,
                                          (hipStream_t)stream);
            if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "spconv_nmap_info");
            const_cast<spconv_nmap*>(h)->valid_pairs = (int64_t)v;
        }
        *valid_pairs = h->valid_pairs;
    }
    return SPCONV_OK;
}

static int forward_impl(const void* feats, int feats_dtype, const spconv_nmap* nmap, const void* w,
                        const void* wpack, const float* bias, void* out, int Ci, int Co, int dtype, void* stream,
                        const char* name, void* cast_ws = nullptr) {
    if (!valid_handle(nmap)) return fail(SPCONV_E_INVALID, "invalid handle");
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16)
        return fail(SPCONV_E_INVALID, "dtype must be SPCONV_F32 or SPCONV_BF16 (got %d)", dtype);
    if (feats_dtype != SPCONV_F32 && feats_dtype != SPCONV_BF16)
        return fail(SPCONV_E_INVALID, "feats_dtype must be SPCONV_F32 or SPCONV_BF16 (got %d)", feats_dtype);
    if (Ci < 1 || Co < 1) return fail(SPCONV_E_INVALID, "Ci and Co must be >= 1");
    if (!spc::forward_supported(dtype, Ci, Co))
        return fail(SPCONV_E_UNSUPPORTED,
                    "no kernel for Ci=%d Co=%d (Ci in {32,64,128,256}, Co a multiple of 32 <= 4096)",
                    Ci, Co);
    if (nmap->N == 0) return SPCONV_OK;
    if (!feats || !w || !out) return fail(SPCONV_E_INVALID, "feats, w and out must be non-NULL");
    if (!aligned(feats, 16) || !aligned(w, 16) || !aligned(out, 16))
        return fail(SPCONV_E_INVALID, "feats, w and out must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SPCONV_E_INVALID, "bias must be 4-byte aligned");
    if (wpack && spc::packed_weight_bytes(nmap->K, Ci, Co, dtype) == 0) wpack = nullptr;  // no packed form
    if (wpack && !aligned(wpack, 16)) return fail(SPCONV_E_INVALID, "wpack must be 16-byte aligned");
    spc::ForwardArgs a;
    a.feats = feats;
    a.nbr_m = nmap->nbr_m;
    a.order = nmap->order;
    a.blkmask = nmap->blkmask;
    a.dcount = nmap->dcount;
    a.drow = nmap->drow;
    a.smap = nmap->smap;
    a.max_distinct = nmap->max_distinct;
    a.w = w;
    a.wpack = wpack;
    a.bias = bias;
    a.out = out;
    a.N = nmap->N;
    a.Npad = nmap->Npad;
    a.K = nmap->K;
    a.Ci = Ci;
    a.Co = Co;
    a.dtype = dtype;
    a.feats_dtype = feats_dtype;
    a.cast_ws = cast_ws;
    // The tile kernel reads w in its packed form only: without one, pack w
    // into a stream-ordered allocation that is released on the stream after
    // the forward.
    hipStream_t st = (hipStream_t)stream;
    void* tmp = nullptr;
    const int fdt = (feats_dtype == SPCONV_F32 && dtype == SPCONV_BF16 && cast_ws) ? SPCONV_BF16 : feats_dtype;
    if (!wpack && spc::tile_forward(dtype, fdt, Ci, Co)) {
        hipError_t e = hipMallocAsync(&tmp, spc::packed_weight_bytes(nmap->K, Ci, Co, dtype), st);
        if (e != hipSuccess) return hip_fail(e, name);
        e = spc::launch_pack_weights(w, nmap->K, Ci, Co, dtype, tmp, st);
        if (e != hipSuccess) {
            (void)hipFreeAsync(tmp, st);
            return hip_fail(e, name);
        }
        a.wpack = tmp;
    }
    hipError_t e = spc::launch_forward(a, st);
    if (tmp) {
        const hipError_t ef = hipFreeAsync(tmp, st);
        if (e == hipSuccess) e = ef;
    }
    return e == hipSuccess ? SPCONV_OK : hip_fail(e, name);
}

int spconv_forward(const void* feats, const spconv_nmap* nmap, const void* w, const float* bias,
                   void* out, int Ci, int Co, int dtype, void* stream) {
    return forward_impl(feats, dtype, nmap, w, nullptr, bias, out, Ci, Co, dtype, stream, "spconv_forward");
}

int spconv_forward_mixed_workspace_size(int64_t N, int Ci, int feats_dtype, int dtype, size_t* bytes) {
    if (!bytes) return fail(SPCONV_E_INVALID, "bytes pointer is NULL");
    if (N < 0 || N > kMaxN) return fail(SPCONV_E_INVALID, "N must be in [0, 2^31-1) (got %lld)", (long long)N);
    if (Ci < 1) return fail(SPCONV_E_INVALID, "Ci must be >= 1");
    if ((feats_dtype != SPCONV_F32 && feats_dtype != SPCONV_BF16) || (dtype != SPCONV_F32 && dtype != SPCONV_BF16))
        return fail(SPCONV_E_INVALID, "feats_dtype and dtype must be SPCONV_F32 or SPCONV_BF16");
    *bytes = spc::cast_workspace_bytes(N, Ci, feats_dtype, dtype);
    return SPCONV_OK;
}

int spconv_forward_mixed(const void* feats, int feats_dtype, const spconv_nmap* nmap, const void* w,
                         const void* wpack, const float* bias, void* out, int Ci, int Co, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_handle(nmap)) return fail(SPCONV_E_INVALID, "invalid handle");
    size_t need = 0;
    int rc = spconv_forward_mixed_workspace_size(nmap->N, Ci, feats_dtype, dtype, &need);
    if (rc) return rc;
    if (need == 0 || nmap->N == 0) workspace = nullptr;   // no cast pass for this pairing
    if (workspace) {
        if (!aligned(workspace, 256)) return fail(SPCONV_E_INVALID, "workspace must be 256-byte aligned");
        if (workspace_bytes < need)
            return fail(SPCONV_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    }
    return forward_impl(feats, feats_dtype, nmap, w, wpack, bias, out, Ci, Co, dtype, stream,
                        "spconv_forward_mixed", workspace);
}

int spconv_pack_weights_size(int K, int Ci, int Co, int dtype, size_t* bytes) {
    if (!bytes) return fail(SPCONV_E_INVALID, "bytes pointer is NULL");
    if (K < 1 || K > kMaxKApi) return fail(SPCONV_E_INVALID, "K must be in [1, %d] (got %d)", kMaxKApi, K);
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16)
        return fail(SPCONV_E_INVALID, "dtype must be SPCONV_F32 or SPCONV_BF16 (got %d)", dtype);
    if (!spc::forward_supported(dtype, Ci, Co))
        return fail(SPCONV_E_UNSUPPORTED, "no kernel for Ci=%d Co=%d", Ci, Co);
    *bytes = spc::packed_weight_bytes(K, Ci, Co, dtype);
    return SPCONV_OK;
}

int spconv_pack_weights(const void* w, int K, int Ci, int Co, int dtype, void* wpack, size_t wpack_bytes,
                        void* stream) {
    size_t need = 0;
    int rc = spconv_pack_weights_size(K, Ci, Co, dtype, &need);
    if (rc) return rc;
    if (need == 0) return SPCONV_OK;
    if (!w || !wpack) return fail(SPCONV_E_INVALID, "w and wpack must be non-NULL");
    if (!aligned(w, 16) || !aligned(wpack, 16)) return fail(SPCONV_E_INVALID, "w and wpack must be 16-byte aligned");
    if (wpack_bytes < need) return fail(SPCONV_E_WORKSPACE, "wpack has %zu bytes, needs %zu", wpack_bytes, need);
    hipError_t e = spc::launch_pack_weights(w, K, Ci, Co, dtype, wpack, (hipStream_t)stream);
    return e == hipSuccess ? SPCONV_OK : hip_fail(e, "spconv_pack_weights");
}


int spconv_forward_packed(const void* feats, const spconv_nmap* nmap, const void* w, const void* wpack,
                          const float* bias, void* out, int Ci, int Co, int dtype, void* stream) {
    if (valid_handle(nmap) && nmap->N > 0 && !wpack && spc::packed_weight_bytes(nmap->K, Ci, Co, dtype) > 0)
        return fail(SPCONV_E_INVALID, "wpack is NULL");
    return forward_impl(feats, dtype, nmap, w, wpack, bias, out, Ci, Co, dtype, stream, "spconv_forward_packed");
}

// Workspace of spconv_dgrad: the mirrored, transposed weights (K x Co x Ci
// elements), then their packed form when the bf16 kernel has one.
static size_t dgrad_wt_bytes(int K, int Ci, int Co, int dtype) {
    return spc::align_up((size_t)K * Ci * Co * (dtype == SPCONV_BF16 ? 2 : 4), 256);
}

int spconv_dgrad_workspace_size(int K, int Ci, int Co, int dtype, size_t* bytes) {
    if (!bytes) return fail(SPCONV_E_INVALID, "bytes pointer is NULL");
    if (K < 1 || K > kMaxKApi) return fail(SPCONV_E_INVALID, "K must be in [1, %d] (got %d)", kMaxKApi, K);
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16)
        return fail(SPCONV_E_INVALID, "dtype must be SPCONV_F32 or SPCONV_BF16 (got %d)", dtype);
    // the gradient runs the forward with the roles of Ci and Co exchanged
    if (!spc::forward_supported(dtype, Co, Ci))
        return fail(SPCONV_E_UNSUPPORTED,
                    "no input-gradient kernel for Ci=%d Co=%d (Co in {32,64,128,256}, Ci a multiple of 32 <= 4096)",
                    Ci, Co);
    *bytes = dgrad_wt_bytes(K, Ci, Co, dtype) + spc::packed_weight_bytes(K, Co, Ci, dtype);
    return SPCONV_OK;
}

int spconv_dgrad(const void* dout, const spconv_nmap* nmap, const void* w, void* workspace,
                 size_t workspace_bytes, void* dfeats, int Ci, int Co, int dtype, void* stream) {
    if (!valid_handle(nmap)) return fail(SPCONV_E_INVALID, "invalid handle");
    if (nmap->wrapped)
        return fail(SPCONV_E_UNSUPPORTED, "the input gradient needs a map from spconv_build_nmap "
                                          "(a caller-made map need not be its own mirror)");
    size_t need = 0;
    int rc = spconv_dgrad_workspace_size(nmap->K, Ci, Co, dtype, &need);
    if (rc) return rc;
    if (nmap->N == 0) return SPCONV_OK;
    if (!w || !workspace) return fail(SPCONV_E_INVALID, "w and workspace must be non-NULL");
    if (!aligned(w, 16) || !aligned(workspace, 256))
        return fail(SPCONV_E_INVALID, "w must be 16-byte and workspace 256-byte aligned");
    if (workspace_bytes < need)
        return fail(SPCONV_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    void* wt = workspace;
    const size_t pk = spc::packed_weight_bytes(nmap->K, Co, Ci, dtype);
    void* wtpack = pk ? (char*)workspace + dgrad_wt_bytes(nmap->K, Ci, Co, dtype) : nullptr;
    hipError_t e = spc::launch_mirror_weights(w, nmap->K, Ci, Co, dtype, wt, (hipStream_t)stream);
    if (e == hipSuccess && wtpack) e = spc::launch_pack_weights(wt, nmap->K, Co, Ci, dtype, wtpack, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "spconv_dgrad");
    return forward_impl(dout, dtype, nmap, wt, wtpack, nullptr, dfeats, Co, Ci, dtype, stream, "spconv_dgrad");
}

int spconv_dgrad_noalloc(const void* dout, const spconv_nmap* nmap, const void* w, void* dfeats, int Ci, int Co,
                         int dtype, void* stream) {
    if (!valid_handle(nmap)) return fail(SPCONV_E_INVALID, "invalid handle");
    size_t need = 0;
    int rc = spconv_dgrad_workspace_size(nmap->K, Ci, Co, dtype, &need);
    if (rc) return rc;
    if (need > kNoAllocScratchBytes)
        return fail(SPCONV_E_WORKSPACE,
                    "spconv_dgrad_noalloc: K=%d Ci=%d Co=%d needs %zu bytes of scratch, beyond its fixed %zu "
                    "(use spconv_dgrad with a workspace)",
                    nmap->K, Ci, Co, need, kNoAllocScratchBytes);
    if (nmap->N == 0) return spconv_dgrad(dout, nmap, w, nullptr, 0, dfeats, Ci, Co, dtype, stream);
    void* ptr = nullptr;
    rc = scratch_address(stream, &ptr, "spconv_dgrad_noalloc");
    if (rc) return rc;
    return spconv_dgrad(dout, nmap, w, ptr, kNoAllocScratchBytes, dfeats, Ci, Co, dtype, stream);
}

int spconv_wgrad_workspace_size(int64_t N, int K, int Ci, int Co, int dtype, size_t* bytes) {
    if (!bytes) return fail(SPCONV_E_INVALID, "bytes pointer is NULL");
    int rc = check_nk(N, K);
    if (rc) return rc;
    if (dtype != SPCONV_F32 && dtype != SPCONV_BF16)
        return fail(SPCONV_E_INVALID, "dtype must be SPCONV_F32 or SPCONV_BF16 (got %d)", dtype);
    if (!spc::wgrad_supported(dtype, Ci, Co))
        return fail(SPCONV_E_UNSUPPORTED, "no weight-gradient kernel for Ci=%d Co=%d (multiples of 32 up to 4096)",
                    Ci, Co);
    *bytes = spc::wgrad_workspace_bytes(N, K, Ci, Co, dtype);
    return SPCONV_OK;
}

int spconv_wgrad(const void* feats, const void* dout, const spconv_nmap* nmap, void* workspace,
                 size_t workspace_bytes, void* dw, int Ci, int Co, int dtype, void* stream) {
    if (!valid_handle(nmap)) return fail(SPCONV_E_INVALID, "invalid handle");
    size_t need = 0;
    int rc = spconv_wgrad_workspace_size(nmap->N, nmap->K, Ci, Co, dtype, &need);
    if (rc) return rc;
    if (!dw) return fail(SPCONV_E_INVALID, "dw is NULL");
    if (!aligned(dw, 16)) return fail(SPCONV_E_INVALID, "dw must be 16-byte aligned");
    if (nmap->N > 0) {
        if (!feats || !dout || !workspace) return fail(SPCONV_E_INVALID, "feats, dout and workspace must be non-NULL");
        if (!aligned(feats, 16) || !aligned(dout, 16) || !aligned(workspace, 256))
            return fail(SPCONV_E_INVALID, "feats and dout must be 16-byte and workspace 256-byte aligned");
        if (workspace_bytes < need)
            return fail(SPCONV_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    }
    spc::WgradArgs a;
    a.feats = feats;
    a.dout = dout;
    a.nbr_m = nmap->nbr_m;
    a.order = nmap->order;
    a.blkmask = nmap->blkmask;
    a.dcount = nmap->dcount;
    a.drow = nmap->drow;
    a.smap = nmap->smap;
    a.max_distinct = nmap->max_distinct;
    a.workspace = workspace;
    a.dw = dw;
    a.N = nmap->N;
    a.Npad = nmap->Npad;
    a.K = nmap->K;
    a.Ci = Ci;
    a.Co = Co;
    a.dtype = dtype;
    // with no rows the gradient is zero (written by the kernels; no workspace used)
    hipError_t e = spc::launch_wgrad(a, (hipStream_t)stream);
    return e == hipSuccess ? SPCONV_OK : hip_fail(e, "spconv_wgrad");
}

void spconv_nmap_destroy(spconv_nmap* h) {
    if (valid_handle(h)) {
        h->magic = 0;
        delete h;
    }
}

}  // extern "C"
