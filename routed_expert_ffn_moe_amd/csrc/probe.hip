// Measurement aids: the ceilings the layer's kernels are compared with on
// the device they run on (not part of the layer's computation).
//
//  probe_read: every CU streams 16-byte non-temporal loads over a buffer
//              (grid-stride, four workgroups per CU, 8 loads in flight per
//              thread) and discards the data: the
//              achievable HBM read rate for a buffer far larger than the
//              caches.
//  probe_gather: the same loads over whole chunks of a pool taken in a
//              given order (one expert's weight block per chunk, the order
//              a seeded shuffle): scattered expert reads, and with a chosen
//              number of workgroups the read rate of a few CUs ("MoE
//              prefill quantum", the section ruling out the hardware: a
//              random read of 300 blocks of 13.3 MB against a sequential
//              one).
//  probe_mxfp4: an MXFP4 dequantisation stream - each thread unpacks 32
//              E2M1 codes of a block, applies its E8M0 scale with the
//              scaled conversion and adds the values up; one float sum per
//              workgroup (the same page and section: unpack x scale +
//              accumulate reads at the raw read rate).
//  probe_mfma: each wave runs 8 independent chains of bf16 16x16x32 MFMAs
//              on register operands: the matrix cores' sustained rate.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int PR_NL = 8;

__global__ __launch_bounds__(256) void probe_read(const uint4 *__restrict__ src, size_t n16,
                                                  int *__restrict__ sink)
{
    uint32_t x = 0;
    const size_t stride = (size_t)gridDim.x * 256 * PR_NL;
    for (size_t base = (size_t)blockIdx.x * 256 * PR_NL + threadIdx.x; base < n16;
         base += stride) {
        uint4 v[PR_NL];
#pragma unroll
        for (int j = 0; j < PR_NL; ++j) {
            const size_t i = base + (size_t)j * 256;
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            // streamed once: non-temporal, as the expert weights are read
            const u32x4 t = i < n16 ? __builtin_nontemporal_load((const u32x4 *)(src + i))
                                    : u32x4{0, 0, 0, 0};
            v[j] = uint4{t[0], t[1], t[2], t[3]};
        }
#pragma unroll
        for (int j = 0; j < PR_NL; ++j)
            x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    if (x == 0x9E3779B9u && sink)  // practically never: keeps the loads
        *sink = (int)x;
}

// Chunk order[c] of the pool (chunk16 16-byte pieces each), walked in
// segments of 256 * PR_NL pieces: segment s is piece (s % per) * 2048 .. of
// the c = s / per-th chunk of the order.
__global__ __launch_bounds__(256) void probe_gather(const uint4 *__restrict__ pool,
                                                    int pool_chunks,
                                                    const int32_t *__restrict__ order, int nchunks,
                                                    size_t chunk16, int *__restrict__ sink)
{
    constexpr size_t SEG = 256 * PR_NL;
    const size_t per = (chunk16 + SEG - 1) / SEG;
    uint32_t x = 0;
    for (size_t s = blockIdx.x; s < (size_t)nchunks * per; s += gridDim.x) {
        const size_t c = s / per, o = (s - c * per) * SEG;  // uniform
        // an order entry outside the pool reads its nearest chunk instead
        const int oc = min(max(order[c], 0), pool_chunks - 1);
        const uint4 *src = pool + (size_t)oc * chunk16;
        uint4 v[PR_NL];
#pragma unroll
        for (int j = 0; j < PR_NL; ++j) {
            const size_t i = o + threadIdx.x + (size_t)j * 256;
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = i < chunk16 ? __builtin_nontemporal_load((const u32x4 *)(src + i))
                                        : u32x4{0, 0, 0, 0};
            v[j] = uint4{t[0], t[1], t[2], t[3]};
        }
#pragma unroll
        for (int j = 0; j < PR_NL; ++j)
            x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    if (x == 0x9E3779B9u && sink)  // practically never: keeps the loads
        *sink = (int)x;
}

// MXFP4 blocks in the OCP row-major form: block b is codes[16 b .. +15]
// (32 E2M1 codes, the even element in the low nibble) and scale byte
// scales[b].  Thread (workgroup w, lane i) takes blocks w * 256 + i,
// then a grid stride further, PR_NL in flight; out[w] = the workgroup's
// sum of its decoded values (fp32, summed per thread, then over threads).
__global__ __launch_bounds__(256) void probe_mxfp4(const uint4 *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales,
                                                   size_t nblocks, float *__restrict__ out)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    float acc = 0.0f;
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t b0 = (size_t)blockIdx.x * 256 + threadIdx.x; b0 < nblocks; b0 += stride * PR_NL) {
        uint4 q[PR_NL];
        uint32_t sc[PR_NL];
#pragma unroll
        for (int j = 0; j < PR_NL; ++j) {
            const size_t b = b0 + (size_t)j * stride;
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = b < nblocks ? __builtin_nontemporal_load((const u32x4 *)(codes + b))
                                        : u32x4{0, 0, 0, 0};
            q[j] = uint4{t[0], t[1], t[2], t[3]};
            sc[j] = b < nblocks ? scales[b] : 0u;
        }
#pragma unroll
        for (int j = 0; j < PR_NL; ++j) {
            // E8M0 s as the exponent field of an fp32: 2^(s - 127)
            const float f = __uint_as_float(sc[j] << 23);
            const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // byte b of the word: elements 2b (low nibble) and 2b + 1
                const f2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], f, 0);
                const f2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], f, 1);
                const f2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], f, 2);
                const f2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], f, 3);
                acc += ((v0[0] + v0[1]) + (v1[0] + v1[1])) + ((v2[0] + v2[1]) + (v3[0] + v3[1]));
            }
        }
    }
    __shared__ float red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h)
            red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        out[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void probe_mfma(int iters, int *__restrict__ sink)
{
    const uint32_t lane = threadIdx.x & 63;
    // operands near 1 (bf16 0x3F80 = 1.0), different per lane
    const uint32_t a0 = 0x3F803F80u + (lane & 7), b0 = 0x3F803F80u + (lane >> 3);
    const bf16x8 a = as_bf16x8(uint4{a0, a0 + 1, a0 + 2, a0 + 3});
    const bf16x8 b = as_bf16x8(uint4{b0, b0 + 1, b0 + 2, b0 + 3});
    floatx4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc[j] = floatx4{0, 0, 0, 0};
    // in place in the accumulation registers (the compiler's own form
    // copies the accumulators out and back every round)
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            mfma16_acc(acc[j], a, b);
    mfma_acc_drain();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (blockIdx.x == 0 && threadIdx.x == 0 && sink)
        *sink = (int)s;
}

}  // namespace

void launch_probe_read(const void *buf, size_t bytes, int *sink, hipStream_t st)
{
    // four workgroups per CU of the 256, 8 loads of 16 bytes in flight per thread
    probe_read<<<1024, 256, 0, st>>>((const uint4 *)buf, bytes / 16, sink);
}

void launch_probe_gather(const void *pool, int pool_chunks, const int32_t *order, int nchunks,
                         size_t chunk_bytes, int wgs, int *sink, hipStream_t st)
{
    probe_gather<<<wgs, 256, 0, st>>>((const uint4 *)pool, pool_chunks, order, nchunks,
                                      chunk_bytes / 16, sink);
}

void launch_probe_mxfp4(const void *codes, const uint8_t *scales, size_t nblocks, int wgs,
                        float *out, hipStream_t st)
{
    probe_mxfp4<<<wgs, 256, 0, st>>>((const uint4 *)codes, scales, nblocks, out);
}

void launch_probe_mfma(int waves, int iters, int *sink, hipStream_t st)
{
    probe_mfma<<<waves / 4, 256, 0, st>>>(iters, sink);
}

}  // namespace moe
