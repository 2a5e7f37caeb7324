/*
 * mlp.h -- C ABI of the fused FP16 MLP inference library for MI355X (gfx950).
 *
 * The operation ("Profiling neural material inference", section "Experiment setup"): one complete
 * evaluation of an affine-layer network per input row, rows independent, about a million rows per
 * dispatch.  Layer l computes y = W_l h + b_l with FP16 weights, biases and activations and an FP32
 * accumulator (the FP16-in / FP32-accumulate convention of "Working with Cooperative Matrices",
 * section "Hardware Constraints and Capabilities"); the FP32 result is rounded to FP16 (nearest,
 * ties to even) and every layer except the last is followed by the leaky ReLU
 * max(v, v * half(0.01)) in FP16 (section "Bad versus good activation").
 *
 * Weights arrive in the canonical FP16 row-major form and are converted once into a device-resident
 * layout before inference, the analogue of the page's one-time conversion to an opaque optimal
 * layout (section "Row-major versus InferencingOptimal weights").  Matrices are tightly packed,
 * stride = number of columns ("Working with Cooperative Matrices", section "Memory Layout").
 *
 * Conventions for every function:
 *   - returns MLP_OK (0) or a negative mlp_status; never aborts, throws or exits;
 *   - argument validation happens on the host before any HIP call, so every validation error is
 *     reported the same way with or without a GPU;
 *   - after an error, mlp_last_error() returns a message for the calling thread;
 *   - "FP16" means IEEE 754 binary16 passed as its 16-bit pattern (uint16_t).
 */
#ifndef MLP_H
#define MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mlp_status {
    MLP_OK = 0,
    MLP_ERR_INVALID_ARGUMENT = -1, /* bad shape, pointer, alignment, enum value or size          */
    MLP_ERR_UNSUPPORTED = -2,      /* valid request that no kernel instance serves                */
    MLP_ERR_NOT_PACKED = -3,       /* mlp_infer before a successful mlp_pack_weights              */
    MLP_ERR_OUT_OF_MEMORY = -4,    /* device allocation failed                                   */
    MLP_ERR_HIP = -5               /* a HIP runtime call failed; the message names it            */
} mlp_status;

/* Weight layouts ("Row-major versus InferencingOptimal weights"). */
enum {
    MLP_LAYOUT_ROW_MAJOR = 0, /* the canonical FP16 row-major matrices, read as they are          */
    MLP_LAYOUT_PACKED = 1,    /* converted once into MFMA-fragment order (the default)            */
    MLP_LAYOUT_PACKED_FP8 = 2 /* the FP8 variant: weights converted once to OCP E4M3 with a       */
                              /* power-of-two scale per output row (the smallest keeping the row  */
                              /* within 448), each layer's input stored as E4M3(16 h), FP32       */
                              /* accumulation, then FP16 rounding and leaky ReLU as in FP16; for  */
                              /* the dedicated shapes and the vector activation                   */
};

/* Activation forms ("Bad versus good activation"); both compute the same function, bit for bit. */
enum {
    MLP_ACT_VECTOR = 0,    /* packed-FP16 max(v, v*half(0.01)) on whole registers (the default)  */
    MLP_ACT_SCALARISED = 1 /* one component at a time: if (v < 0) v *= half(0.01)                */
};

#define MLP_MAX_LAYERS 64  /* any network up to 64 layers ...                                  */
#define MLP_MAX_WIDTH 4096 /* ... of widths up to 4096 (see MLP_FUSED_*)                         */
/* Networks within these limits run as one fused kernel (weights in LDS, activations in registers):
 * up to MLP_FUSED_MAX_LAYERS layers of widths up to MLP_FUSED_MAX_WIDTH, or up to
 * MLP_FUSED_DEEP_MAX_LAYERS layers with the input width a multiple of 8 and the output width of 4:
 * always when every width is at most 64, and at widths up to 128 unless the layer-by-layer path
 * runs the whole network as one chain (every layer padded to 128 outputs, the input width a multiple
 * of 64, the output width of 8), which is faster there.  Wider or deeper ones run layer by layer (one
 * MFMA GEMM with the fused epilogue per layer, the activations between layers in device memory; a
 * run of layers of equal width class, at most 64, at most 128 or 256 padded outputs, as one launch
 * with the activations kept in LDS), packed layout and vector activation only. */
#define MLP_FUSED_MAX_LAYERS 8
#define MLP_FUSED_MAX_WIDTH 128
#define MLP_FUSED_DEEP_MAX_LAYERS 16

/* Size in bytes of the device image mlp_pack_weights would build for this shape and layout: the
 * size query that precedes the one-time conversion ("Row-major versus InferencingOptimal weights":
 * the application asks for the converted matrix's size before converting into it).
 *   n_layers  number of affine layers, 1..MLP_MAX_LAYERS
 *   widths    n_layers + 1 entries: widths[0] = input width, widths[l] = output width of layer l,
 *             each 1..MLP_MAX_WIDTH
 *   layout    MLP_LAYOUT_ROW_MAJOR, MLP_LAYOUT_PACKED or MLP_LAYOUT_PACKED_FP8
 *   out_bytes receives the size
 * Host only; no HIP call.  MLP_ERR_UNSUPPORTED for a row-major request on a shape that no dedicated
 * kernel serves (generic fused shapes and layer-by-layer shapes take the packed layout only). */
int mlp_packed_size(int n_layers, const int32_t *widths, int layout, size_t *out_bytes);

/* The widths the selected kernel computes with (input width padded as the kernel reads it, every
 * layer width padded to its tile multiple, except that a last layer of at most 4 outputs on a
 * dedicated FP16 kernel is computed 4 wide): kernel_widths receives n_layers + 1 entries.  Shapes
 * without a dedicated kernel but within the fused limits run on a generic fused kernel whose widths
 * are all 64 (when every width is at most 64) or all MLP_FUSED_MAX_WIDTH, zero-padded; wider or
 * deeper shapes run layer by layer with the input width padded to a multiple of 64 and every layer
 * width to a multiple of 128.
 * Host only; no HIP call. */
int mlp_plan_widths(int n_layers, const int32_t *widths, int layout, int32_t *kernel_widths);

/* Build the device image into a caller-owned host buffer of dst_bytes (>= mlp_packed_size).
 *   weights   n_layers host pointers; weights[l] is [widths[l+1]][widths[l]] FP16 row-major
 *   biases    n_layers host pointers; biases[l] is [widths[l+1]] FP16
 * Host only; no HIP call.  Used by tests and by callers that manage device memory themselves. */
int mlp_pack_host(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                  const uint16_t *const *biases, int layout, void *host_dst, size_t dst_bytes);

/* One-time conversion: pack the weights (same arguments as mlp_pack_host) and upload them to the
 * current HIP device.  This becomes the library's current network, replacing any previous one.
 *   stream    hipStream_t for the upload (NULL = the default stream); the call synchronises it
 *             before returning, so the caller may free weights and biases afterwards.
 * Ownership: the library owns the device image until mlp_release or the next successful pack.
 * Not thread-safe; do not re-pack while an mlp_infer on the previous network may still run.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, OUT_OF_MEMORY, HIP (previous network kept on error). */
int mlp_pack_weights(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                     const uint16_t *const *biases, int layout, void *stream);

/* The same one-time conversion from weights already resident on the device, run as a kernel on
 * `stream` ("Row-major versus InferencingOptimal weights": the conversion can be recorded into the
 * GPU's command stream instead of run on the host).  The resulting device image is bit for bit the
 * one mlp_pack_weights builds, and it becomes the current network.
 *   layout    MLP_LAYOUT_PACKED (every shape, fused or layer by layer), MLP_LAYOUT_ROW_MAJOR or
 *             MLP_LAYOUT_PACKED_FP8 (the dedicated shapes; the kernel computes each row's scale and
 *             rounds to E4M3 exactly as the host packer does)
 *   d_weights n_layers host-memory entries, each a device pointer to [widths[l+1]][widths[l]] FP16
 *             row-major, 2-byte aligned
 *   d_biases  n_layers host-memory entries, each a device pointer to [widths[l+1]] FP16
 *   stream    hipStream_t (NULL = the default stream) the conversion is enqueued on
 * Stream-ordered: the call allocates the image, enqueues the conversion and returns without waiting.
 * When the current network's image has the same size on the same device and n_layers <= 16, the
 * conversion rewrites that image in place instead (no allocation, no free, nothing that waits for the
 * device): work already enqueued on `stream` still sees the previous network, and no mlp_infer on
 * another stream may be running on it (as for any re-pack).
 * The weights must stay valid, and unchanged, until the stream has run the conversion; an
 * mlp_infer on the same stream sees the converted image, one on another stream must first wait for
 * this stream (e.g. with an event).  Ownership, threading and errors as for mlp_pack_weights, except
 * that a device-side fault surfaces at the caller's next synchronisation. */
int mlp_pack_weights_device(int n_layers, const int32_t *widths, const void *const *d_weights,
                            const void *const *d_biases, int layout, void *stream);

/* Evaluate the current network on `batch` rows: enqueue one kernel on `stream` and return.  This is
 * the timed inference pass of "Profiling neural material inference", section "Experiment setup" (one
 * dispatch evaluates every row through every layer); per layer y = W h + b in FP32 from FP16
 * operands, rounded to FP16, then max(v, v * half(0.01)) except after the last layer (section "Bad
 * versus good activation").
 *   batch    number of rows, >= 0 (0: nothing is launched, returns MLP_OK)
 *   in_ptr   device pointer, [batch][widths[0]] FP16 row-major, 16-byte aligned
 *   out_ptr  device pointer, [batch][widths[n_layers]] FP16 row-major, 16-byte aligned, must not
 *            overlap in_ptr
 *   stream   hipStream_t (NULL = the default stream)
 * Asynchronous: the buffers must stay valid until the stream's work completes.  A network beyond the
 * fused limits runs as one kernel per layer over blocks of rows (as many as make the scratch below
 * 512 MiB, at least 65,536), its intermediate activations in two scratch buffers (block rows x the
 * widest hidden width, padded to 64, FP16) that the call allocates and frees in order on `stream`
 * from a memory pool the library keeps (so calls on different streams never share them);
 * MLP_ERR_OUT_OF_MEMORY if they cannot be allocated.  Must be called with the device that was
 * current at pack time.  Uses the activation form set by
 * mlp_set_activation_mode (default MLP_ACT_VECTOR).  Concurrent calls on different streams are
 * safe (the weights are read-only).  A device fault, should one occur, surfaces at the caller's
 * next synchronisation, as with any HIP kernel.
 * Errors: INVALID_ARGUMENT, NOT_PACKED, UNSUPPORTED, HIP (launch failure). */
int mlp_infer(int64_t batch, const void *in_ptr, void *out_ptr, void *stream);

/* mlp_infer for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, semantics and errors as mlp_infer,
 * but it calls no hipMalloc, hipFree or pool allocation.  A fused network (the dedicated and generic
 * kernels) uses no scratch memory, so there it runs exactly what mlp_infer runs.  A network beyond the
 * fused limits keeps its intermediate activations in a fixed scratch array of 64 MiB per GPU (file-
 * scope device memory, looked up on the first call on each device and held until the process ends)
 * instead of the pool: rows run in blocks of as many row tiles (256 rows) as two blocks of activations
 * at the widest hidden layer (padded to 64, FP16) fit in 64 MiB, e.g. 16,384 rows at width 1024 and
 * 4,096 rows at width 4096; MLP_ERR_UNSUPPORTED if not even one row tile fits (never, within
 * MLP_MAX_WIDTH).  The array keeps the last call's contents; every value a call reads from it was
 * written earlier in the same call, so nothing needs clearing.  All calls on one GPU share that
 * array: two calls whose work may overlap on the GPU (different streams, or different threads on the
 * same stream without ordering) race on it and may corrupt each other's results; order them, e.g.
 * one stream or events. */
int mlp_infer_noalloc(int64_t batch, const void *in_ptr, void *out_ptr, void *stream);

/* mlp_infer with an explicit activation form (MLP_ACT_VECTOR or MLP_ACT_SCALARISED). */
int mlp_infer_ex(int64_t batch, const void *in_ptr, void *out_ptr, void *stream, int act_mode);

/* Set the activation form mlp_infer uses (process-wide).  For A/B measurement. */
int mlp_set_activation_mode(int act_mode);

/* Name of the kernel instance that serves the current network with the given activation form,
 * written NUL-terminated into buf (at most buf_bytes bytes, truncated if needed). */
int mlp_kernel_name(int act_mode, char *buf, size_t buf_bytes);

/* Copy the current device image back to host memory (bytes must equal its size).  For tests. */
int mlp_debug_read_packed(void *host_dst, size_t bytes);

/* Message for the last error on the calling thread ("" if none).  Valid until the next call. */
const char *mlp_last_error(void);

/* Free the current device image (the converted matrices of "Row-major versus InferencingOptimal
 * weights", which live until the weights change) and return the scratch memory the layer-by-layer
 * path keeps cached
 * (its stream-ordered frees complete first).  Idempotent; mlp_infer then returns MLP_ERR_NOT_PACKED.
 * Not thread-safe with respect to mlp_pack_weights or an mlp_infer still being enqueued. */
void mlp_release(void);

#ifdef __cplusplus
}
#endif

#endif /* MLP_H */
