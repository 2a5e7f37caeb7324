// mlp_api.cpp -- the C ABI declared in include/mlp.h: validation, library state, HIP plumbing.
//
// Every argument is validated on the host before the first HIP call.  The library holds one packed
// network (the current net) on the device that was current when it was packed.
#include <hip/hip_runtime.h>  // HIP_SYMBOL and __device__ for the no-alloc scratch array
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "mlp.h"
#include "mlp_testing.h"
#include "mlp_layered.h"
#include "mlp_layout.h"
#include "mlp_pack.h"
#include "mlp_registry.h"

using mlpk::KernelEntry;

namespace {

thread_local std::string t_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_error = buf;
    return code;
}

int ok()
{
    t_error.clear();
    return MLP_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(MLP_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

struct State {
    bool packed = false;
    int n_layers = 0;
    int widths[MLP_MAX_LAYERS + 1] = {};
    int layout = MLP_LAYOUT_PACKED;
    const KernelEntry *entry[2] = {nullptr, nullptr};  // per activation form
    int grid_cap[2] = {0, 0};
    int cus = 0;  // compute units of the device
    void *image = nullptr;
    size_t bytes = 0;
    int device = -1;
};

State g_net;
int g_act_mode = MLP_ACT_VECTOR;

// The layer-by-layer path (mlp_layered.hip) stands in the registry's place for shapes no fused kernel
// serves: widths above MLP_FUSED_MAX_WIDTH, more than MLP_FUSED_DEEP_MAX_LAYERS layers, or more than
// MLP_FUSED_MAX_LAYERS without vector I/O or, at widths above 64, when one chain serves the network.
const KernelEntry kLayered = {"mlp_layered<256/128/64-wide chains | gemm 256x256 | 128x256, fused epilogue>", 0, {}, true, MLP_LAYOUT_PACKED,
                              MLP_ACT_VECTOR, 256, 64, true, nullptr, nullptr};
bool is_layered(const KernelEntry *e) { return e == &kLayered; }

// Rows per pass of the layered path: as many as two blocks of activations at the widest hidden
// layer fit in kLayeredScratchBytes, and at least kLayeredMinRows.  Larger passes mean fewer
// launches, each with more workgroups than the GPU holds at once (a launch of one round of
// workgroups pays a whole tail).
constexpr int64_t kLayeredMinRows = 65536;
constexpr int64_t kLayeredScratchBytes = (int64_t)512 << 20;

// Device memory for the layered path's intermediate activations: a pool owned by the library with
// no release threshold, so that the stream-ordered allocation of each call reuses memory.
hipMemPool_t g_pool = nullptr;
int g_pool_device = -1;
std::mutex g_pool_mu;  // mlp_infer may be called from several threads at once

int layered_pool(int device, hipMemPool_t *out)
{
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (!g_pool || g_pool_device != device) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = device;
        hipMemPool_t pool = nullptr;
        hipError_t err = hipMemPoolCreate(&pool, &props);
        if (err != hipSuccess)
            return hip_fail(err, "hipMemPoolCreate");
        uint64_t keep = UINT64_MAX;
        err = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (err != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return hip_fail(err, "hipMemPoolSetAttribute(release threshold)");
        }
        g_pool = pool;  // a pool made for another device is kept: its memory may still be in use
        g_pool_device = device;
    }
    *out = g_pool;
    return MLP_OK;
}

size_t state_image_bytes(int n_layers, const int32_t *widths, int layout, const KernelEntry *e)
{
    return is_layered(e) ? mlpk::layered_image_bytes(n_layers, widths) : mlpk::image_bytes(n_layers, e->widths, layout);
}

int check_shape(int n_layers, const int32_t *widths)
{
    if (n_layers < 1 || n_layers > MLP_MAX_LAYERS)
        return fail(MLP_ERR_INVALID_ARGUMENT, "n_layers must be in [1, %d], got %d", MLP_MAX_LAYERS, n_layers);
    if (!widths)
        return fail(MLP_ERR_INVALID_ARGUMENT, "widths is NULL");
    for (int i = 0; i <= n_layers; ++i)
        if (widths[i] < 1 || widths[i] > MLP_MAX_WIDTH)
            return fail(MLP_ERR_INVALID_ARGUMENT, "widths[%d] = %d is outside [1, %d]", i, (int)widths[i], MLP_MAX_WIDTH);
    return MLP_OK;
}

int check_layout(int layout)
{
    if (layout != MLP_LAYOUT_ROW_MAJOR && layout != MLP_LAYOUT_PACKED && layout != MLP_LAYOUT_PACKED_FP8)
        return fail(MLP_ERR_INVALID_ARGUMENT, "unknown layout %d", layout);
    return MLP_OK;
}

int check_act(int act)
{
    if (act != MLP_ACT_VECTOR && act != MLP_ACT_SCALARISED)
        return fail(MLP_ERR_INVALID_ARGUMENT, "unknown activation mode %d", act);
    return MLP_OK;
}

// The instance that serves (shape, layout, act): an exact-shape instance, else for the packed
// layout with the vector activation and widths within the fused limits the first generic instance
// for that layer count that serves the shape: padded widths that cover it and, for the vector-I/O
// family, an input width that is a multiple of 8 and an output width that is a multiple of 4 (the
// registry lists the 64-wide families before the 128-wide one), else none.
const KernelEntry *select(int n_layers, const int32_t *widths, int layout, int act)
{
    int count = 0;
    const KernelEntry *all = mlpk::registry(&count);
    if (layout == MLP_LAYOUT_PACKED_FP8) {  // dedicated shapes only
        all = mlpk::registry_fp8(&count);
        if (act != MLP_ACT_VECTOR)
            return nullptr;
    }
    for (int i = 0; i < count; ++i) {
        const KernelEntry &e = all[i];
        if (e.generic || e.n_layers != n_layers || e.layout != layout || e.act != act)
            continue;
        bool same = true;
        for (int k = 0; k <= n_layers; ++k)
            same &= e.widths[k] == widths[k];
        if (same)
            return &e;
    }
    if (layout != MLP_LAYOUT_PACKED || act != MLP_ACT_VECTOR)
        return nullptr;
    for (int k = 0; k <= n_layers; ++k)
        if (widths[k] > MLP_FUSED_MAX_WIDTH)
            return nullptr;  // beyond the generic kernels
    for (int i = 0; i < count; ++i) {
        if (!all[i].generic || all[i].n_layers != n_layers)
            continue;
        bool covers = true;
        for (int k = 0; k <= n_layers; ++k)
            covers &= widths[k] <= all[i].widths[k];
        if (all[i].vec_io && (widths[0] % 8 != 0 || widths[n_layers] % 4 != 0))
            covers = false;  // its vector loads and stores need these widths
        if (n_layers > MLP_FUSED_MAX_LAYERS && all[i].widths[0] > 64 && mlpk::layered_one_narrow_chain(n_layers, widths))
            covers = false;  // a deep 128-wide net that one chain serves runs faster layer by layer
        if (covers)
            return &all[i];
    }
    return nullptr;
}

int plan(int n_layers, const int32_t *widths, int layout, const KernelEntry **out)
{
    int rc = check_shape(n_layers, widths);
    if (rc == MLP_OK)
        rc = check_layout(layout);
    if (rc != MLP_OK)
        return rc;
    const KernelEntry *e = select(n_layers, widths, layout, MLP_ACT_VECTOR);
    if (!e && layout == MLP_LAYOUT_PACKED)
        e = &kLayered;  // wider or deeper than the fused kernels
    if (!e)
        return fail(MLP_ERR_UNSUPPORTED, "no kernel serves this shape with the %s layout (row-major and FP8 are "
                    "compiled for the dedicated shapes only)",
                    layout == MLP_LAYOUT_PACKED ? "packed" : layout == MLP_LAYOUT_ROW_MAJOR ? "row-major" : "FP8");
    *out = e;
    return MLP_OK;
}

int check_weights(int n_layers, const uint16_t *const *weights, const uint16_t *const *biases)
{
    if (!weights || !biases)
        return fail(MLP_ERR_INVALID_ARGUMENT, "weights or biases is NULL");
    for (int l = 0; l < n_layers; ++l)
        if (!weights[l] || !biases[l])
            return fail(MLP_ERR_INVALID_ARGUMENT, "weights[%d] or biases[%d] is NULL", l, l);
    return MLP_OK;
}

}  // namespace

extern "C" {

int mlp_packed_size(int n_layers, const int32_t *widths, int layout, size_t *out_bytes)
{
    if (!out_bytes)
        return fail(MLP_ERR_INVALID_ARGUMENT, "out_bytes is NULL");
    const KernelEntry *e = nullptr;
    const int rc = plan(n_layers, widths, layout, &e);
    if (rc != MLP_OK)
        return rc;
    *out_bytes = state_image_bytes(n_layers, widths, layout, e);
    return ok();
}

int mlp_plan_widths(int n_layers, const int32_t *widths, int layout, int32_t *kernel_widths)
{
    if (!kernel_widths)
        return fail(MLP_ERR_INVALID_ARGUMENT, "kernel_widths is NULL");
    const KernelEntry *e = nullptr;
    const int rc = plan(n_layers, widths, layout, &e);
    if (rc != MLP_OK)
        return rc;
    if (is_layered(e)) {
        kernel_widths[0] = mlpk::layered_kin(widths[0]);
        for (int l = 1; l <= n_layers; ++l)
            kernel_widths[l] = mlpk::layered_kout(widths[l]);
        return ok();
    }
    kernel_widths[0] = mlpl::k0_pad(e->widths[0]);
    for (int l = 1; l <= n_layers; ++l)
        kernel_widths[l] = mlpl::round_up(e->widths[l], mlpl::kTileM);
    if (layout != MLP_LAYOUT_PACKED_FP8 && mlpl::narrow_last(e->widths, n_layers))
        kernel_widths[n_layers] = mlpl::kNarrowOut;  // the 16x16x32 form: 4 outputs per sample half
    return ok();
}

int mlp_pack_host(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                  const uint16_t *const *biases, int layout, void *host_dst, size_t dst_bytes)
{
    const KernelEntry *e = nullptr;
    int rc = plan(n_layers, widths, layout, &e);
    if (rc == MLP_OK)
        rc = check_weights(n_layers, weights, biases);
    if (rc != MLP_OK)
        return rc;
    const size_t need = state_image_bytes(n_layers, widths, layout, e);
    if (!host_dst)
        return fail(MLP_ERR_INVALID_ARGUMENT, "host_dst is NULL");
    if (dst_bytes < need)
        return fail(MLP_ERR_INVALID_ARGUMENT, "host_dst holds %zu bytes, the image needs %zu", dst_bytes, need);
    if (is_layered(e))
        mlpk::pack_layered(n_layers, widths, weights, biases, (uint8_t *)host_dst);
    else
        mlpk::pack_image(n_layers, widths, e->widths, weights, biases, layout, (uint8_t *)host_dst);
    return ok();
}

}  // extern "C"

namespace {

// A new State for (shape, layout) served by `e`, with its device image allocated (contents unset).
// reuse_image: take the current network's image instead when it has the same size on the same device
// (the caller then rewrites it in place, in stream order, with no allocation and no free).
int new_state(int n_layers, const int32_t *widths, int layout, const KernelEntry *e, State &next,
              bool reuse_image = false)
{
    next.n_layers = n_layers;
    for (int i = 0; i <= n_layers; ++i)
        next.widths[i] = widths[i];
    next.layout = layout;
    next.entry[MLP_ACT_VECTOR] = e;
    next.entry[MLP_ACT_SCALARISED] = is_layered(e) ? nullptr : select(n_layers, widths, layout, MLP_ACT_SCALARISED);
    next.bytes = state_image_bytes(n_layers, widths, layout, e);
    hipError_t err = hipGetDevice(&next.device);
    if (err != hipSuccess)
        return hip_fail(err, "hipGetDevice");
    int cus = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, next.device);
    if (err != hipSuccess)
        return hip_fail(err, "hipDeviceGetAttribute(multiProcessorCount)");
    next.cus = cus;
    for (int a = 0; a < 2; ++a) {
        const KernelEntry *k = next.entry[a];
        if (!k || is_layered(k))
            continue;
        int blocks = 0;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k->func, k->threads, 0);
        if (err != hipSuccess)
            return hip_fail(err, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
        if (blocks < 1)
            return fail(MLP_ERR_UNSUPPORTED, "kernel %s cannot be resident on this device", k->name);
        next.grid_cap[a] = blocks * cus;
    }
    if (reuse_image && g_net.packed && g_net.device == next.device && g_net.bytes == next.bytes) {
        next.image = g_net.image;
        return MLP_OK;
    }
    err = hipMalloc(&next.image, next.bytes);
    if (err != hipSuccess) {
        next.image = nullptr;
        const int code = err == hipErrorOutOfMemory ? MLP_ERR_OUT_OF_MEMORY : MLP_ERR_HIP;
        return fail(code, "hipMalloc(%zu) failed: %s", next.bytes, hipGetErrorString(err));
    }
    return MLP_OK;
}

void commit_state(State &next)
{
    next.packed = true;
    if (g_net.packed && g_net.image != next.image)
        (void)hipFree(g_net.image);
    g_net = next;
}

}  // namespace

extern "C" {

int mlp_pack_weights(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                     const uint16_t *const *biases, int layout, void *stream)
{
    const KernelEntry *e = nullptr;
    int rc = plan(n_layers, widths, layout, &e);
    if (rc == MLP_OK)
        rc = check_weights(n_layers, weights, biases);
    if (rc != MLP_OK)
        return rc;
    std::vector<uint8_t> host(state_image_bytes(n_layers, widths, layout, e));
    if (is_layered(e))
        mlpk::pack_layered(n_layers, widths, weights, biases, host.data());
    else
        mlpk::pack_image(n_layers, widths, e->widths, weights, biases, layout, host.data());

    State next;
    rc = new_state(n_layers, widths, layout, e, next);
    if (rc != MLP_OK)
        return rc;
    hipError_t err = hipMemcpyAsync(next.image, host.data(), next.bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (err == hipSuccess)
        err = hipStreamSynchronize((hipStream_t)stream);
    if (err != hipSuccess) {
        (void)hipFree(next.image);
        return hip_fail(err, "uploading the weight image");
    }
    commit_state(next);
    return ok();
}

int mlp_testing_plan_kernel(int n_layers, const int32_t *widths, int layout, char *name, size_t cap)
{
    const KernelEntry *e = nullptr;
    const int rc = plan(n_layers, widths, layout, &e);
    if (rc != MLP_OK)
        return rc;
    if (!name || cap == 0)
        return fail(MLP_ERR_INVALID_ARGUMENT, "name is NULL or empty");
    snprintf(name, cap, "%s", e->name);
    return ok();
}

int mlp_testing_pack_device_on_host(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                                    const uint16_t *const *biases, int layout, void *host_dst, size_t dst_bytes,
                                    int *exact_cover)
{
    const KernelEntry *e = nullptr;
    int rc = plan(n_layers, widths, layout, &e);
    if (rc == MLP_OK)
        rc = check_weights(n_layers, weights, biases);
    if (rc != MLP_OK)
        return rc;
    const size_t need = state_image_bytes(n_layers, widths, layout, e);
    if (!host_dst || !exact_cover)
        return fail(MLP_ERR_INVALID_ARGUMENT, "host_dst or exact_cover is NULL");
    if (dst_bytes != need)
        return fail(MLP_ERR_INVALID_ARGUMENT, "host_dst holds %zu bytes, the image has %zu", dst_bytes, need);
    std::vector<uint8_t> written(need, 0);
    bool clean = true;
    for (int l0 = 0; l0 < n_layers; l0 += mlpk::kPackMaxLayers) {  // as mlp_pack_weights_device launches it
        const int count = n_layers - l0 < mlpk::kPackMaxLayers ? n_layers - l0 : mlpk::kPackMaxLayers;
        mlpk::PackArgs args{};
        if (is_layered(e))
            mlpk::fill_pack_args_layered(widths, l0, count, args);
        else
            mlpk::fill_pack_args(n_layers, widths, e->widths, layout, args);
        for (int i = 0; i < count; ++i) {
            args.w[i] = weights[l0 + i];
            args.b[i] = biases[l0 + i];
        }
        clean &= mlpk::pack_items_on_host(args, count, (uint8_t *)host_dst, need, written);
    }
    for (size_t k = 0; k < need && clean; ++k)
        clean = written[k] == 1;
    *exact_cover = clean ? 1 : 0;
    return ok();
}

int mlp_pack_weights_device(int n_layers, const int32_t *widths, const void *const *d_weights,
                            const void *const *d_biases, int layout, void *stream)
{
    const KernelEntry *e = nullptr;
    int rc = plan(n_layers, widths, layout, &e);
    if (rc == MLP_OK)
        rc = check_weights(n_layers, (const uint16_t *const *)d_weights, (const uint16_t *const *)d_biases);
    if (rc != MLP_OK)
        return rc;
    for (int l = 0; l < n_layers; ++l)
        if (((uintptr_t)d_weights[l] | (uintptr_t)d_biases[l]) & 1)
            return fail(MLP_ERR_INVALID_ARGUMENT, "d_weights[%d] or d_biases[%d] is not 2-byte aligned", l, l);
    // One launch (at most 16 layers) rewrites an image of unchanged size in place: hipFree would wait for
    // the whole device, and a conversion recorded into the stream should not.  Deeper networks take
    // several launches and a new image, so a failed launch never leaves the current network half
    // rewritten.
    State next;
    rc = new_state(n_layers, widths, layout, e, next, n_layers <= mlpk::kPackMaxLayers);
    if (rc != MLP_OK)
        return rc;
    // The conversion kernel takes up to kPackMaxLayers layers per launch (a fused network in one).
    for (int l0 = 0; l0 < n_layers; l0 += mlpk::kPackMaxLayers) {
        const int count = n_layers - l0 < mlpk::kPackMaxLayers ? n_layers - l0 : mlpk::kPackMaxLayers;
        mlpk::PackArgs args{};
        if (is_layered(e))
            mlpk::fill_pack_args_layered(widths, l0, count, args);
        else
            mlpk::fill_pack_args(n_layers, widths, e->widths, layout, args);
        for (int i = 0; i < count; ++i) {
            args.w[i] = (const uint16_t *)d_weights[l0 + i];
            args.b[i] = (const uint16_t *)d_biases[l0 + i];
        }
        args.dst = (uint8_t *)next.image;
        const hipError_t err = mlpk::launch_pack(args, count, (hipStream_t)stream);
        if (err != hipSuccess) {
            if (next.image != g_net.image)
                (void)hipFree(next.image);
            return hip_fail(err, "launching the device packer");
        }
    }
    commit_state(next);
    return ok();
}

}  // extern "C"

namespace {

// The scratch array of mlp_infer_noalloc: file-scope device memory, one copy per GPU, held until the
// process ends.  Host code never uses its name as an address: each device's address is looked up once
// (hipGetSymbolAddress, with that device current) and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// This device's scratch address; looked up on the device's first call.  `device` must be current.
int scratch_address(int device, void **out)
{
    if (device < 0 || device >= kMaxDevices)
        return fail(MLP_ERR_UNSUPPORTED, "device %d is beyond the %d devices mlp_infer_noalloc tracks", device, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *ptr = nullptr;
        const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return hip_fail(err, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return MLP_OK;
}

// The layered path: rows in blocks, each block through every layer, with the activations between
// layers in two scratch buffers.  Without `ext` the buffers are allocated on the stream (stream-ordered,
// so calls on different streams never share them) and freed on it afterwards, with blocks as large as
// kLayeredScratchBytes allows (at least kLayeredMinRows); with `ext` (ext_bytes of caller-provided
// device memory) nothing is allocated and the blocks are as large as `ext` holds.
int infer_layered(int64_t batch, const void *in_ptr, void *out_ptr, hipStream_t stream, void *ext = nullptr,
                  size_t ext_bytes = 0)
{
    const int L = g_net.n_layers;
    const int *w = g_net.widths;
    int ld_max = 0;  // row stride of the scratch buffers: the widest hidden layer, padded to 64 halves
    for (int l = 1; l < L; ++l)
        ld_max = mlpk::layered_kin(w[l]) > ld_max ? mlpk::layered_kin(w[l]) : ld_max;
    const int64_t tile = mlpk::layered_rows_per_tile();
    const int64_t row_bytes = 2 * 2 * (int64_t)(ld_max > 0 ? ld_max : 1);  // both buffers, FP16
    int64_t block = kLayeredScratchBytes / row_bytes / tile * tile;
    block = block > kLayeredMinRows ? block : kLayeredMinRows;
    if (ext) {
        block = (int64_t)ext_bytes / row_bytes / tile * tile;
        if (block < tile)
            return fail(MLP_ERR_UNSUPPORTED, "one row tile of this network's activations needs %lld bytes, more than "
                        "the %zu bytes of mlp_infer_noalloc's scratch", (long long)(tile * row_bytes), ext_bytes);
    }
    const int64_t chunk = batch < block ? batch : block;
    void *buf[2] = {nullptr, nullptr};
    if (ext) {
        buf[0] = ext;
        buf[1] = (uint8_t *)ext + (size_t)chunk * ld_max * 2;  // chunk: a multiple of the tile, or the batch
    } else if (L > 1) {
        hipMemPool_t pool = nullptr;
        const int rc = layered_pool(g_net.device, &pool);
        if (rc != MLP_OK)
            return rc;
        const size_t bytes = (size_t)chunk * ld_max * 2;
        for (int i = 0; i < (L > 2 ? 2 : 1); ++i) {
            const hipError_t err = hipMallocFromPoolAsync(&buf[i], bytes, pool, stream);
            if (err != hipSuccess) {
                if (buf[0])
                    (void)hipFreeAsync(buf[0], stream);
                const int code = err == hipErrorOutOfMemory ? MLP_ERR_OUT_OF_MEMORY : MLP_ERR_HIP;
                return fail(code, "hipMallocFromPoolAsync(%zu) failed: %s", bytes, hipGetErrorString(err));
            }
        }
    }
    hipError_t err = hipSuccess;
    for (int64_t r0 = 0; r0 < batch && err == hipSuccess; r0 += chunk) {
        const int64_t rows = batch - r0 < chunk ? batch - r0 : chunk;
        // layer j's input and output rows in this block
        auto x_of = [&](int j) { return j == 0 ? (const uint16_t *)in_ptr + r0 * w[0] : (const uint16_t *)buf[(j - 1) & 1]; };
        auto ldx_of = [&](int j) { return (int64_t)(j == 0 ? w[0] : ld_max); };
        auto y_of = [&](int j) { return j == L - 1 ? (uint16_t *)out_ptr + r0 * w[L] : (uint16_t *)buf[j & 1]; };
        auto ldy_of = [&](int j) { return (int64_t)(j == L - 1 ? w[L] : ld_max); };
        for (int l = 0; l < L && err == hipSuccess;) {
            // A chain [l, e): layers that run at one chain width (all 256; or 128 and 64, at 64 when
            // every layer is of class 64), the first reading whole 16-byte rows of exactly its K
            // columns, the last writing 16-byte rows of a multiple of 8 outputs.
            const int k0 = mlpk::layered_chain_class(w[l], w[l + 1]);
            int e = l;
            while (k0 && e < L && e - l < mlpk::kChainMaxLayers &&
                   mlpk::layered_chain_joins(k0, mlpk::layered_chain_class(w[e], w[e + 1])))
                ++e;
            while (e - l >= 2 && !(w[e] % 8 == 0 && ldy_of(e - 1) % 8 == 0 && ((uintptr_t)y_of(e - 1) & 15) == 0))
                --e;
            int cw = 0;
            for (int j = l; j < e; ++j)
                cw = std::max(cw, mlpk::layered_chain_class(w[j], w[j + 1]));
            const bool whole_x = w[l] == mlpk::layered_kin(w[l]) && ldx_of(l) % 8 == 0 && ((uintptr_t)x_of(l) & 15) == 0;
            if (e - l >= 2 && whole_x) {
                mlpk::ChainArgs c{};
                c.x = x_of(l);
                c.ldx = ldx_of(l);
                c.y = y_of(e - 1);
                c.ldy = ldy_of(e - 1);
                c.width = cw;
                c.wout_last = w[e];
                c.image = (const uint8_t *)g_net.image;
                c.rows = rows;
                c.row_tiles = (rows + 255) / 256;
                c.n = e - l;
                c.act_last = e < L;
                for (int j = l; j < e; ++j) {
                    c.off[j - l] = mlpk::layered_layer_offset(w, j);
                    c.kin[j - l] = mlpk::layered_kin(w[j]);
                }
                err = mlpk::launch_chain(c, stream);
                l = e;
                continue;
            }
            mlpk::LayerArgs a{};
            a.x = x_of(l);
            a.ldx = ldx_of(l);
            a.y = y_of(l);
            a.ldy = ldy_of(l);
            const size_t off = mlpk::layered_layer_offset(w, l);
            a.a = (const uint8_t *)g_net.image + off;
            a.bias = (const float *)((const uint8_t *)g_net.image + off + mlpk::layered_a_bytes(w[l], w[l + 1]));
            a.rows = rows;
            a.row_tiles = (rows + mlpk::layered_rows_per_tile() - 1) / mlpk::layered_rows_per_tile();
            a.win = w[l];
            a.wout = w[l + 1];
            a.kin = mlpk::layered_kin(w[l]);
            a.kout = mlpk::layered_kout(w[l + 1]);
            a.act = l + 1 < L;
            a.vec_x = a.ldx % 8 == 0 && ((uintptr_t)a.x & 15) == 0;
            a.vec_y = a.ldy % 4 == 0 && ((uintptr_t)a.y & 7) == 0;
            a.cus = g_net.cus;
            err = mlpk::launch_layer(a, stream);
            ++l;
        }
    }
    if (!ext)
        for (int i = 0; i < 2; ++i)
            if (buf[i])
                (void)hipFreeAsync(buf[i], stream);
    if (err != hipSuccess)
        return hip_fail(err, "layer kernel launch");
    return ok();
}

// mlp_infer_ex and mlp_infer_noalloc: validation, then the fused kernel or the layered path.
int infer(int64_t batch, const void *in_ptr, void *out_ptr, void *stream, int act_mode, bool noalloc)
{
    if (batch < 0)
        return fail(MLP_ERR_INVALID_ARGUMENT, "batch must be >= 0, got %lld", (long long)batch);
    int rc = check_act(act_mode);
    if (rc != MLP_OK)
        return rc;
    if (!g_net.packed)
        return fail(MLP_ERR_NOT_PACKED, "no network: call mlp_pack_weights first");
    const KernelEntry *e = g_net.entry[act_mode];
    if (!e)
        return fail(MLP_ERR_UNSUPPORTED, "the %s activation form is compiled for the dedicated shapes only",
                    act_mode == MLP_ACT_SCALARISED ? "scalarised" : "vector");
    if (batch == 0)
        return ok();
    const int w0 = g_net.widths[0], wL = g_net.widths[g_net.n_layers];
    if (batch > INT64_MAX / (2 * MLP_MAX_WIDTH))
        return fail(MLP_ERR_INVALID_ARGUMENT, "batch %lld is too large", (long long)batch);
    if (!in_ptr || !out_ptr)
        return fail(MLP_ERR_INVALID_ARGUMENT, "in_ptr or out_ptr is NULL");
    if (((uintptr_t)in_ptr | (uintptr_t)out_ptr) & 15)
        return fail(MLP_ERR_INVALID_ARGUMENT, "in_ptr and out_ptr must be 16-byte aligned");
    const uintptr_t i0 = (uintptr_t)in_ptr, i1 = i0 + (uintptr_t)(batch * w0 * 2);
    const uintptr_t o0 = (uintptr_t)out_ptr, o1 = o0 + (uintptr_t)(batch * wL * 2);
    if (i0 < o1 && o0 < i1)
        return fail(MLP_ERR_INVALID_ARGUMENT, "in and out buffers overlap");

    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return hip_fail(err, "hipGetDevice");
    if (dev != g_net.device)
        return fail(MLP_ERR_INVALID_ARGUMENT, "current device %d is not the device %d the network was packed on",
                    dev, g_net.device);

    if (is_layered(e)) {
        if (!noalloc)
            return infer_layered(batch, in_ptr, out_ptr, (hipStream_t)stream);
        void *ptr = nullptr;
        rc = scratch_address(dev, &ptr);
        if (rc != MLP_OK)
            return rc;
        return infer_layered(batch, in_ptr, out_ptr, (hipStream_t)stream, ptr, kNoAllocScratchBytes);
    }
    const int64_t rows_per_block = (int64_t)e->rows_per_wave * (e->threads / 64);
    const int64_t blocks = (batch + rows_per_block - 1) / rows_per_block;
    const int grid = (int)(blocks < g_net.grid_cap[act_mode] ? blocks : g_net.grid_cap[act_mode]);
    mlpk::LaunchArgs a;
    a.x = (const uint16_t *)in_ptr;
    a.y = (uint16_t *)out_ptr;
    a.image = (const uint8_t *)g_net.image;
    a.batch = batch;
    a.w0 = w0;
    a.wL = wL;
    err = e->launch(a, grid, (hipStream_t)stream);
    if (err != hipSuccess)
        return hip_fail(err, "kernel launch");
    return ok();
}

}  // namespace

extern "C" {

int mlp_infer_ex(int64_t batch, const void *in_ptr, void *out_ptr, void *stream, int act_mode)
{
    return infer(batch, in_ptr, out_ptr, stream, act_mode, false);
}

int mlp_infer_noalloc(int64_t batch, const void *in_ptr, void *out_ptr, void *stream)
{
    return infer(batch, in_ptr, out_ptr, stream, g_act_mode, true);
}

int mlp_infer(int64_t batch, const void *in_ptr, void *out_ptr, void *stream)
{
    return mlp_infer_ex(batch, in_ptr, out_ptr, stream, g_act_mode);
}

int mlp_set_activation_mode(int act_mode)
{
    const int rc = check_act(act_mode);
    if (rc != MLP_OK)
        return rc;
    g_act_mode = act_mode;
    return ok();
}

int mlp_kernel_name(int act_mode, char *buf, size_t buf_bytes)
{
    int rc = check_act(act_mode);
    if (rc != MLP_OK)
        return rc;
    if (!buf || buf_bytes == 0)
        return fail(MLP_ERR_INVALID_ARGUMENT, "buf is NULL or empty");
    if (!g_net.packed)
        return fail(MLP_ERR_NOT_PACKED, "no network: call mlp_pack_weights first");
    const KernelEntry *e = g_net.entry[act_mode];
    if (!e)
        return fail(MLP_ERR_UNSUPPORTED, "no kernel for this activation form on the current network");
    snprintf(buf, buf_bytes, "%s", e->name);
    return ok();
}

int mlp_debug_read_packed(void *host_dst, size_t bytes)
{
    if (!g_net.packed)
        return fail(MLP_ERR_NOT_PACKED, "no network: call mlp_pack_weights first");
    if (!host_dst || bytes != g_net.bytes)
        return fail(MLP_ERR_INVALID_ARGUMENT, "need a host buffer of exactly %zu bytes", g_net.bytes);
    const hipError_t err = hipMemcpy(host_dst, g_net.image, bytes, hipMemcpyDeviceToHost);
    if (err != hipSuccess)
        return hip_fail(err, "hipMemcpy(device image -> host)");
    return ok();
}

const char *mlp_last_error(void) { return t_error.c_str(); }

void mlp_release(void)
{
    {
        // hand the layered path's cached scratch memory back (pending frees complete first)
        std::lock_guard<std::mutex> lock(g_pool_mu);
        if (g_pool)
            (void)hipMemPoolTrimTo(g_pool, 0);
    }
    if (g_net.packed)
        (void)hipFree(g_net.image);
    g_net = State();
}

}  // extern "C"
