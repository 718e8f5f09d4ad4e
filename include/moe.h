/*
 * moe.h - C ABI of the MI355X (gfx950) routed-expert MoE FFN layer library
 * (libmoe.so).
 *
 * The layer, for every token t of x[T, H]:
 *   1. router: logits l = x_t . router_w^T (+ router_bias), accumulated in
 *      fp32 and never rounded to bf16; the top_k experts by logit (descending,
 *      ties to the lower expert index); weights w = softmax of the k selected
 *      logits (equal to the full softmax renormalised over the selection).
 *      Pages: "MoE prefill quantum" (cause section: each token uses k of E
 *      experts); "DeepSeek V4.1F Q4 with native DSpark MTP" (decode
 *      paragraph: the router as a single fused dispatch).
 *   2. permutation: the (t, j) pairs grouped by expert, stably (t, then j
 *      ascending within an expert).
 *   3. per expert e: h = silu(x W_gate[e]^T) * (x W_up[e]^T)  (SwiGLU with the
 *      SiLU on the gate branch; "Jetson Orin Nano MoE ... expert cache",
 *      re-check section and gate-first section).
 *   4. o = h W_down[e]^T, scaled by w[t, j]; y_t = sum over j = 0..k-1 of the
 *      scaled rows in that fixed order (same page, nondeterminism section:
 *      each expert owns its output rows, so the order of the sum is fixed),
 *      plus, if present, the always-on shared expert's output with weight 1
 *      ("DeepSeek V4.1F" decode paragraph).
 *
 * Layouts (row-major, K-contiguous):
 *   x [T, H], y [T, H]              act_dtype (MOE_F32 or MOE_BF16)
 *   router_w [E, H]                 act_dtype
 *   router_bias [E]                 float, or NULL
 *   w_gate, w_up [E, I, H]          w_dtype
 *   w_down [E, H, I]                w_dtype
 *     MXFP4 (OCP MX v1.0): the matrices as moe_pack_mxfp4 lays them out
 *     (below), from the OCP row-major form: codes [E, N, K/2], two E2M1
 *     codes per byte, even element in the low nibble, and E8M0 scales
 *     [E, N, K/32], one per 32 consecutive K elements ([N, K] = [I, H] for
 *     gate and up, [H, I] for down).
 *   sh_gate, sh_up [I_shared, H], sh_down [H, I_shared]   act_dtype
 *     BF16 expert matrices (routed and shared) are passed as moe_pack_bf16
 *     lays them out (below); F32 ones row-major as listed.  The caller
 *     states which in moe_weights_t.layout: MOE_LAYOUT_PACKED is required for
 *     BF16 and MXFP4 expert matrices, MOE_LAYOUT_ROWMAJOR for F32 ones; any
 *     other combination is refused with MOE_EINVAL (a zero-initialised
 *     struct says ROWMAJOR, so row-major bf16 weights never reach a kernel).
 *   topk_idx [T, top_k] int32, topk_w [T, top_k] float
 *
 * Packed MXFP4 (what the kernels read: each wave's weights are whole
 * contiguous kilobytes).  Rows go in blocks of 16 (n = 16*nb + r) and K in
 * steps of 128 (q = K/128 steps); the lane index l = r + 16*b, b = 0..3:
 *   codes  [E][N/16][q][64 lanes][16 B]: lane l of step s holds the 32 codes
 *          of row n at K = 128*s + 32*b .. +31 (OCP byte order);
 *   scales [E][N/16][64 lanes][q]: byte s of lane l is the scale of row n
 *          at K = 128*s + 32*b .. +31.
 * The packed matrices have the same sizes as the OCP ones.
 *
 * Packed BF16 (what the kernels read: a wave's weight fragment of one MFMA
 * step is a contiguous kilobyte).  Rows go in groups of 32 (g = n / 32) and
 * K in steps of 32 (s = k / 32); each (g, s) is two 1 KB blocks c = 0, 1;
 * lane l = r + 16*b (r = 0..15, b = 0..3) of block c holds the 8 elements
 * of row n = 32*g + 8*(r/4) + 4*c + r%4 at K = 32*s + 8*b .. +7:
 *   [E][N/32][K/32][2][64 lanes][8 bf16].
 *
 * Supported combinations: act F32 with w F32; act BF16 with w BF16 or MXFP4.
 * MXFP4 needs H and I multiples of 128, at most 4096, and no shared expert
 * (MOE_EINVAL / MOE_EUNSUPPORTED otherwise).  One pass (chunk) of Tc tokens
 * must keep Tc * H, Tc * E * 8 and rows * max(H, I, I_shared) below 2^31,
 * rows = Tc * top_k (+ Tc with a shared expert); larger passes are refused
 * with MOE_EINVAL (split them with chunk_T).
 * Every pointer except router_bias, topk_w and the unused ones is a device
 * pointer, 16-byte aligned.  The caller owns all memory; the library
 * allocates nothing per call and keeps no state between calls other than
 * cached device properties.  Calls are asynchronous on `stream` (a
 * hipStream_t, NULL = the default stream): outputs are valid once the stream
 * has synchronised.  Nothing is read back to the host inside a call.
 *
 * Error handling: every entry point returns MOE_OK (0) or a negative code;
 * no exception crosses the boundary.  On MOE_EINVAL / MOE_EWORKSPACE nothing
 * has been launched.  On MOE_EHIP a launch failed; moe_last_error() gives the
 * HIP error text of the calling thread's last failure.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype_t;

/* Layout of the expert matrices in moe_weights_t (see Layouts above). */
enum { MOE_LAYOUT_ROWMAJOR = 0, MOE_LAYOUT_PACKED = 1 };

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* null/misaligned pointer, bad size or dtype  */
    MOE_EWORKSPACE = -2,   /* ws_bytes < moe_workspace_bytes(shape)       */
    MOE_EUNSUPPORTED = -3, /* device is not gfx950, or dtype combination  */
    MOE_EHIP = -4          /* HIP launch/runtime error                    */
};

/* Sizes of one call.
 *  - top_k is a run-time value, not a property of the weights: a caller may
 *    run a layer with fewer experts per token than it was trained with ("Jetson
 *    Orin Nano MoE: GPU clock floor and expert cache", section on decode time
 *    as a fixed part plus a read part, where the model's experts-per-token
 *    count is overridden from 8 to 4).
 *  - chunk_T is the prefill quantum: the number of tokens the layer is handed
 *    at a time ("MoE prefill quantum", the one-line summary and the inverse
 *    equation quantum = target tokens per expert x E / top_k).  Passes of
 *    chunk_T tokens run one after the other on one workspace; tokens are
 *    independent, so y does not depend on it. */
typedef struct {
    int32_t T;         /* tokens                                             */
    int32_t H;         /* hidden size (multiple of 64)                       */
    int32_t E;         /* routed experts, 1..1023                            */
    int32_t top_k;     /* experts per token, 1..min(E, 16)                   */
    int32_t I;         /* expert intermediate size (multiple of 64)          */
    int32_t I_shared;  /* shared expert intermediate size, 0 = none          */
    int32_t chunk_T;   /* tokens per internal pass, 0 = all T at once        */
    int32_t act_dtype; /* moe_dtype_t of x, y, router_w and shared weights   */
    int32_t w_dtype;   /* moe_dtype_t of the routed expert weights           */
} moe_shape_t;

typedef struct {
    const void *router_w;
    const float *router_bias;                /* nullable                     */
    const void *w_gate, *w_up, *w_down;      /* codes when w_dtype == MXFP4  */
    const uint8_t *s_gate, *s_up, *s_down;   /* E8M0, MXFP4 only             */
    const void *sh_gate, *sh_up, *sh_down;   /* I_shared > 0 only            */
    int32_t layout;  /* MOE_LAYOUT_* of the expert and shared matrices       */
} moe_weights_t;

/* Bytes of device workspace moe_forward / moe_route need for `shape`
 * (sized for one chunk of min(T, chunk_T) tokens); 0 if the shape is
 * invalid. */
size_t moe_workspace_bytes(const moe_shape_t *shape);

/* The whole layer: y [T, H] and the routing (topk_idx required, topk_w
 * nullable).  The routing is returned because callers keep it: per-layer
 * logs of the experts the router chose are what an expert cache's policy is
 * chosen from ("Jetson Orin Nano MoE: GPU clock floor and expert cache",
 * section on choosing what to cache from the router's records).  `ws` is device memory of at least moe_workspace_bytes(shape)
 * bytes, 256-byte aligned, owned by the caller; its contents on entry do not
 * matter.  The result does not depend on chunk_T beyond rounding order: each
 * chunk is processed independently in token order. */
int moe_forward(const moe_shape_t *shape, const moe_weights_t *w,
                const void *x, void *y, int32_t *topk_idx, float *topk_w,
                void *ws, size_t ws_bytes, void *stream);

/* Bytes of the static device scratch moe_forward_noalloc uses (per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that must not call
 * hipMalloc.  Same arguments and results as moe_forward, without the
 * workspace: the scratch comes from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds
 * from the library's first use there until the process ends; its address on
 * a device is looked up on the first call on that device.  Allocates nothing
 * (no hipMalloc/hipFree, no allocating library routine).  A shape whose pass
 * (min(T, chunk_T) tokens) needs more scratch than that is refused with
 * MOE_EWORKSPACE before anything is launched (moe_workspace_bytes gives the
 * need; a smaller chunk_T lowers it: 52 MiB for 1024 tokens at H=2048, E=256,
 * top-8, I=768).  Every call on a GPU shares that GPU's scratch and leaves
 * its contents behind (no call needs it cleared): calls that overlap on one
 * GPU, from several streams or threads, race. */
int moe_forward_noalloc(const moe_shape_t *shape, const moe_weights_t *w,
                        const void *x, void *y, int32_t *topk_idx, float *topk_w,
                        void *stream);

/* Router and permutation only (analysis / test export).  For the tokens of
 * one pass (chunk_T must be 0 or >= T): topk_idx [T, k], topk_w [T, k],
 * counts [E] (pairs per expert), offsets [E+1] (exclusive prefix of counts)
 * and row_src [T*k] (the pair t*k+j at each grouped position).  All device
 * pointers; topk_w, counts, offsets and row_src are nullable. */
int moe_route(const moe_shape_t *shape, const moe_weights_t *w,
              const void *x, int32_t *topk_idx, float *topk_w,
              int32_t *counts, int32_t *offsets, int32_t *row_src,
              void *ws, size_t ws_bytes, void *stream);

/* Repack E MXFP4 matrices of N rows and K columns (N a multiple of 16, K of
 * 128) from the OCP row-major form (codes [E, N, K/2], scales [E, N, K/32])
 * into the layout moe_forward reads (above); E * N * K / 2 code bytes and
 * E * N * K / 32 scale bytes out.  Device pointers, 16-byte aligned, the
 * outputs not overlapping the inputs; asynchronous on `stream`.  A one-time
 * step when weights are loaded.  MOE_EINVAL on bad sizes or pointers. */
int moe_pack_mxfp4(int E, int N, int K, const void *codes, const uint8_t *scales,
                   void *codes_out, uint8_t *scales_out, void *stream);

/* Repack E bf16 matrices of N rows and K columns (multiples of 32) from the
 * row-major form [E, N, K] into the layout moe_forward reads (above); the
 * same number of bytes out.  Device pointers, 16-byte aligned, not
 * overlapping; asynchronous on `stream`.  A one-time step when weights are
 * loaded.  MOE_EINVAL on bad sizes or pointers. */
int moe_pack_bf16(int E, int N, int K, const void *w, void *w_out, void *stream);

/* Stage timing for measurement (not needed for computing).  While enabled,
 * moe_forward records a pair of HIP events on its stream around each of its
 * stages - 0 router, 1 permutation, 2 gate+up, 3 down, 4 combine - for up to
 * 4096 calls; moe_stage_timing_read waits for them, writes the summed
 * milliseconds per stage into ms[0..n_stages) and the number of recorded
 * calls into *n_calls, and clears the record.  Enabling or disabling also
 * clears it.  Process-wide; returns MOE_OK or MOE_EHIP. */
int moe_stage_timing_enable(int on);
int moe_stage_timing_read(float *ms, int n_stages, int *n_calls);

/* Measurement aids (not part of the layer): the ceilings its kernels are
 * compared with on this device.  Asynchronous on `stream`; time them with
 * events around the call.
 * moe_probe_read reads `bytes` (a positive multiple of 16) at the device
 * pointer buf with 16-byte loads from every CU and discards the data, so a
 * buffer much larger than the caches gives the achievable HBM read rate.
 * moe_probe_mfma runs `iters` rounds of 8 independent bf16 16x16x32 MFMA
 * chains in each of `waves` waves (a positive multiple of 4): 8 * 16384
 * floating-point operations per wave and round, the matrix cores' sustained
 * bf16 rate.  sink is a device int (or NULL) that may receive a value
 * derived from the results.  MOE_EINVAL for bad sizes or a NULL buffer,
 * MOE_EHIP if the launch fails. */
int moe_probe_read(const void *buf, size_t bytes, void *stream);
int moe_probe_mfma(int waves, int iters, int *sink, void *stream);

/* Scattered expert-block reads ("MoE prefill quantum", the section ruling
 * out the hardware, which times a random read of 300 blocks of 13.3 MB
 * beside a sequential read).  pool: a device buffer of pool_bytes holding
 * pool_bytes / chunk_bytes chunks of chunk_bytes (a positive multiple of 16;
 * one expert's weight block); order: a device int32 array of nchunks chunk
 * numbers (entries outside the pool read the nearest chunk); the chunks are
 * read whole in that order by `wgs` workgroups of 256 threads (1..65536;
 * fewer workgroups than CUs gives the read rate of that many CUs), 16-byte
 * non-temporal loads, data discarded: nchunks * chunk_bytes bytes.
 * moe_probe_mxfp4 streams nblocks MXFP4 blocks in the OCP row-major form
 * (codes: 16 bytes per block, 32 E2M1 codes, the even element in the low
 * nibble, 16-byte aligned; scales: one E8M0 byte per block), decodes every
 * value as code x 2^(scale - 127) with the scaled fp4 conversion and adds
 * them up: out[w] (a device float array of wgs entries) receives workgroup
 * w's fp32 sum, so the stream is checkable; 17/32 byte per value ("MoE
 * prefill quantum", the same section: unpacking and scaling MXFP4 streams
 * at the raw read rate).  Both asynchronous on `stream`; MOE_EINVAL for bad
 * sizes or NULL / misaligned pointers (checked before any launch), MOE_EHIP
 * if the launch fails. */
int moe_probe_gather(const void *pool, size_t pool_bytes, size_t chunk_bytes,
                     const int32_t *order, int nchunks, int wgs, void *stream);
int moe_probe_mxfp4(const void *codes, const uint8_t *scales, size_t nblocks, int wgs,
                    float *out, void *stream);

/* Static text for a return code. */
const char *moe_strerror(int code);

/* Detail of the calling thread's last failure (argument name or HIP error). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
