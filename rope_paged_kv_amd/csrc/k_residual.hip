// Residual update of a frame's hidden states after an attention layer, fused
// with the cast that feeds the next layer's projection: x += o in fp32, then
// xb = bf16(x).  Page "How LingBot-Map Achieves Real-Time 3D Reconstruction",
// section "AggregatorStream with FlashInfer Paged KV Cache": every frame and
// global block adds its attention output back into the token stream.
//
// HBM-bound: per element 4 B of x read and written, 2 B of o read, 2 B of xb
// written (12 B).  One thread per 8 elements: two 16-byte loads of x, one of
// o, two 16-byte stores of x and one of xb, all coalesced; a ragged tail of
// fewer than 8 elements is done one element per thread by the last
// workgroup.
#include "rpkv_internal.h"

namespace rpkv {

namespace {

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ inline uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__global__ __launch_bounds__(256) void k_residual_add(float* __restrict__ x,
                                                       const uint16_t* __restrict__ o,
                                                       uint16_t* __restrict__ xb, long long n8,
                                                       int tail) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n8) {
        float4* xp = reinterpret_cast<float4*>(x) + 2 * i;
        const uint4 ov = reinterpret_cast<const uint4*>(o)[i];
        float4 a = xp[0], b = xp[1];
        a.x += bf16_value(ov.x & 0xFFFFu);
        a.y += bf16_value(ov.x >> 16);
        a.z += bf16_value(ov.y & 0xFFFFu);
        a.w += bf16_value(ov.y >> 16);
        b.x += bf16_value(ov.z & 0xFFFFu);
        b.y += bf16_value(ov.z >> 16);
        b.z += bf16_value(ov.w & 0xFFFFu);
        b.w += bf16_value(ov.w >> 16);
        xp[0] = a;
        xp[1] = b;
        if (xb) {
            uint4 r;
            r.x = bf16_bits(a.x) | (bf16_bits(a.y) << 16);
            r.y = bf16_bits(a.z) | (bf16_bits(a.w) << 16);
            r.z = bf16_bits(b.x) | (bf16_bits(b.y) << 16);
            r.w = bf16_bits(b.z) | (bf16_bits(b.w) << 16);
            reinterpret_cast<uint4*>(xb)[i] = r;
        }
    }
    // the last workgroup also takes the tail (threads 0 .. tail-1)
    if (blockIdx.x == gridDim.x - 1 && (int)threadIdx.x < tail) {
        const long long j = 8 * n8 + threadIdx.x;
        const float v = x[j] + bf16_value(o[j]);
        x[j] = v;
        if (xb) xb[j] = (uint16_t)bf16_bits(v);
    }
}

}  // namespace

hipError_t launch_residual_add(float* x, const uint16_t* o, uint16_t* xb, long long n,
                               hipStream_t st) {
    const long long n8 = n / 8;
    const int tail = (int)(n - 8 * n8);
    const long long blocks = n8 > 0 ? (n8 + 255) / 256 : 1;
    hipLaunchKernelGGL(k_residual_add, dim3((unsigned)blocks), dim3(256), 0, st, x, o, xb, n8, tail);
    return hipGetLastError();
}

}  // namespace rpkv
