// Paged attention of one frame's tokens over the visible page table.
//
// What is computed (page "How 3D RoPE Positional Encoding Works with the Paged
// KV Cache in LingBot-Map", section "Attention Computation with Cached RoPE";
// page "How LingBot-Map Achieves Real-Time 3D Reconstruction", section
// "Per-Frame Processing and Causal Attention"): for every query token i of the
// frame and head h, softmax(q_i . k_j / sqrt(D)) weighted sum of v_j over the
// visible keys j -- the patch tokens of the visible patch pages (scale pages,
// window pages, the frame's own page) and the tokens of the visible special
// pages, the last one holding last_page_len tokens.  K is already rotated in
// the cache, so nothing positional is recomputed here.
//
// This file: the dispatcher, the merge of key-range splits and the fp32
// kernel (a plain per-query loop in fp32 on the FMA units).  The bf16
// matrix-core kernel is in k_attend_bf16.hip.
#include "rpkv_internal.h"

namespace rpkv {

template <typename T>
__device__ inline void tile_ref(const AttnArgs& a, int s, int h, int t, int n_patch_tiles,
                                const int* vis, const int* vis_len, int vis_sp, const T*& k,
                                const T*& v, int& vstride, int& len) {
    if (t < n_patch_tiles) {
        const int pi = t / a.tpp;
        const int off = (t - pi * a.tpp) * kTile;
        const int page = vis[pi];
        const size_t pg = (size_t)h * a.pool + page;
        k = (const T*)a.kpool + s * a.kpool_elems + (pg * a.slot_cap + off) * kHeadDim;
        v = (const T*)a.vpool + s * a.kpool_elems + pg * kHeadDim * a.slot_cap + off;
        vstride = a.slot_cap;
        len = min(kTile, vis_len[pi] - off);   // a page holds the tokens its frame had
    } else {
        const int off = (t - n_patch_tiles) * kTile;
        k = (const T*)a.ksp + s * a.ksp_elems + ((size_t)h * a.sp_cap + off) * kHeadDim;
        v = (const T*)a.vsp + s * a.ksp_elems + (size_t)h * kHeadDim * a.sp_cap + off;
        vstride = a.sp_cap;
        len = min(kTile, vis_sp - off);
    }
}

// Merge of the key-range splits: out = sum_i w_i O_i / sum_i w_i with
// w_i = exp(lse_i - max lse); lse = max + log(sum w).  Split i's partial
// output arrives as fp16 words scaled by a power of two and the fp32 factor
// f_i that undoes it (O_i = f_i * words), beside its LSE.  One thread per
// (stream, head, query, 8 channels): 16-byte loads of the words, and both
// split loops unrolled so that their loads are in flight together (the merge
// is latency-bound otherwise: a few bytes per thread per split).
template <typename T>
__global__ __launch_bounds__(256) void k_attend_combine(AttnArgs a) {
    const size_t idx = blockIdx.x * (size_t)256 + threadIdx.x;
    const size_t total = (size_t)a.S * a.H * a.N * 8;
    if (idx >= total) return;
    const int d8 = idx & 7;
    const size_t rest = idx >> 3;
    const int q = rest % a.N;
    const int sh = rest / a.N;   // s*H + h
    const int s = sh / a.H, h = sh % a.H;
    if (q >= a.states[s].n_query) return;   // not a token of this frame
    const size_t base = (size_t)sh * a.splits * a.N + q;
    float mx = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < a.splits; ++i) mx = fmaxf(mx, a.part_ls[base + (size_t)i * a.N].x);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
    if (mx > -INFINITY) {
#pragma unroll 4
        for (int i = 0; i < a.splits; ++i) {
            const size_t row = base + (size_t)i * a.N;
            const float2 ls = a.part_ls[row];
            const uint4 u = *(const uint4*)(a.part_o + row * kHeadDim + d8 * 8);   // 8 fp16
            const float w = __expf(ls.x - mx);
            const float wf = w * ls.y;
            const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += wf * (float)__builtin_bit_cast(_Float16, (uint16_t)(uw[e] & 0xFFFFu));
                acc[2 * e + 1] += wf * (float)__builtin_bit_cast(_Float16, (uint16_t)(uw[e] >> 16));
            }
            wsum += w;
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    T* op = (T*)a.out + (((size_t)s * a.N + q) * a.H + h) * kHeadDim + d8 * 8;
    if constexpr (sizeof(T) == 2) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 lo = (__bf16)(acc[2 * e] * inv);
            const __bf16 hi = (__bf16)(acc[2 * e + 1] * inv);
            w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *(uint4*)op = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        *(float4*)op = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        *(float4*)(op + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
    if (d8 == 0 && a.lse) a.lse[(size_t)sh * a.N + q] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

// fp32: one query per thread, fp32 throughout (precise exp/log).
__global__ __launch_bounds__(64) void k_attend_f32(AttnArgs a) {
    __shared__ float ks[kTile][kHeadDim + 1];
    __shared__ float vs[kHeadDim][kTile + 1];
    const int h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
    const CacheState* st = a.states + s;
    const int q = blockIdx.x * 64 + tid;
    const bool qvalid = q < st->n_query;
    const int vis_n = st->vis_n, vis_sp = st->vis_sp_tokens;
    const int n_patch_tiles = vis_n * a.tpp;
    const int n_tiles = n_patch_tiles + (vis_sp + kTile - 1) / kTile;

    float qr[kHeadDim], o[kHeadDim];
    const float* qp = (const float*)a.q + (((size_t)s * a.N + (qvalid ? q : 0)) * a.H + h) * kHeadDim;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) {
        qr[d] = qvalid ? qp[d] : 0.f;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int t = 0; t < n_tiles; ++t) {
        const float* kp;
        const float* vp;
        int vstride, len;
        tile_ref<float>(a, s, h, t, n_patch_tiles, st->vis, st->vis_len, vis_sp, kp, vp, vstride, len);
        __syncthreads();
        // 16-byte loads, all issued before the LDS stores: thread tid takes
        // float4 chunks tid, tid+64, ... of the K tile and of the V^T tile.
        float4 kr[16], vr[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = tid + 64 * j;          // chunk: row i/16, columns 4*(i%16)..+3
            kr[j] = *(const float4*)(kp + (size_t)(i >> 4) * kHeadDim + 4 * (i & 15));
            vr[j] = *(const float4*)(vp + (size_t)(i >> 4) * vstride + 4 * (i & 15));
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = tid + 64 * j, r = i >> 4, c4 = 4 * (i & 15);
            ks[r][c4] = kr[j].x;
            ks[r][c4 + 1] = kr[j].y;
            ks[r][c4 + 2] = kr[j].z;
            ks[r][c4 + 3] = kr[j].w;
            vs[r][c4] = vr[j].x;
            vs[r][c4 + 1] = vr[j].y;
            vs[r][c4 + 2] = vr[j].z;
            vs[r][c4 + 3] = vr[j].w;
        }
        __syncthreads();
        for (int j = 0; j < len; ++j) {
            float sdot = 0.f;
#pragma unroll
            for (int d = 0; d < kHeadDim; ++d) sdot = fmaf(qr[d], ks[j][d], sdot);
            sdot *= a.scale;
            const float m_new = fmaxf(m, sdot);
            const float alpha = expf(m - m_new);
            const float p = expf(sdot - m_new);
            l = l * alpha + p;
            const int pos = vslot_perm(j);
#pragma unroll
            for (int d = 0; d < kHeadDim; ++d) o[d] = fmaf(p, vs[d][pos], o[d] * alpha);
            m = m_new;
        }
    }
    if (!qvalid) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = (float*)a.out + (((size_t)s * a.N + q) * a.H + h) * kHeadDim;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) op[d] = o[d] * inv;
    if (a.lse) a.lse[((size_t)s * a.H + h) * a.N + q] = l > 0.f ? m + logf(l) : -INFINITY;
}

hipError_t launch_attend(const AttnArgs& a, int dtype, hipStream_t st) {
    if (dtype == RPKV_F32) {
        dim3 grid((a.N + 63) / 64, a.H, a.S);
        hipLaunchKernelGGL(k_attend_f32, grid, dim3(64), 0, st, a);
        return hipGetLastError();
    }
    hipError_t e = launch_attend_bf16_main(a, st);
    if (e != hipSuccess || a.splits == 1) return e;
    const size_t total = (size_t)a.S * a.H * a.N * 8;
    hipLaunchKernelGGL(k_attend_combine<uint16_t>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace rpkv
