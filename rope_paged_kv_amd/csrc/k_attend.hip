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
// bf16 path (matrix cores, gfx950 v_mfma_f32_32x32x16_bf16):
//  * a workgroup of 4 waves takes 128 queries of one (stream, head) and one
//    split of the visible key range; each wave owns 32 queries;
//  * keys are walked in tiles of 64 that never straddle a page: a patch page of
//    P tokens is ceil(P/64) tiles, the special stream (contiguous in token
//    order, pages appended in order) is another ceil(n/64); K and V^T tiles are
//    staged through double-buffered LDS by all 256 threads;
//  * scores are formed transposed, S^T = K Q^T (keys on the MFMA rows,
//    queries on the columns), so every lane holds 32 scores of one query:
//    the running max and the row sum stay in-lane but for one exchange with the
//    lane 32 apart; P^T converted to bf16 is directly the B operand of
//    O^T = V^T P^T, with V stored transposed in the cache in the key order
//    the score layout produces;
//  * online softmax in base 2 with the 1/sqrt(D)*log2(e) factor folded into
//    one FMA, fp32 accumulation;
//  * several splits of the key range are merged by their log-sum-exp.
// fp32 path: a plain per-query loop in fp32 (FMA units), same tiles.
#include "rpkv_internal.h"

namespace rpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kQW = 32;                 // queries per wave
constexpr int kQB = kWaves * kQW;       // queries per workgroup
constexpr int kLds = kHeadDim + 8;      // LDS row stride (elements): 144 B, staggers banks

struct TileRef {
    const uint16_t* k;   // 64 rows of D elements
    const uint16_t* v;   // D rows of 64 positions, row stride vstride
    int vstride;
    int len;             // valid keys in the tile (1..64)
};

template <typename T>
__device__ inline void tile_ref(const AttnArgs& a, int s, int h, int t, int n_patch_tiles,
                                const int* vis, int vis_sp, const T*& k, const T*& v,
                                int& vstride, int& len) {
    if (t < n_patch_tiles) {
        const int pi = t / a.tpp;
        const int off = (t - pi * a.tpp) * kTile;
        const int page = vis[pi];
        const size_t pg = (size_t)h * a.pool + page;
        k = (const T*)a.kpool + s * a.kpool_elems + (pg * a.slot_cap + off) * kHeadDim;
        v = (const T*)a.vpool + s * a.kpool_elems + pg * kHeadDim * a.slot_cap + off;
        vstride = a.slot_cap;
        len = min(kTile, a.P - off);
    } else {
        const int off = (t - n_patch_tiles) * kTile;
        k = (const T*)a.ksp + s * a.ksp_elems + ((size_t)h * a.sp_cap + off) * kHeadDim;
        v = (const T*)a.vsp + s * a.ksp_elems + (size_t)h * kHeadDim * a.sp_cap + off;
        vstride = a.sp_cap;
        len = min(kTile, vis_sp - off);
    }
}

// Walks the tiles of one split in order: patch pages (tpp tiles each), then
// the special stream.  Addresses advance incrementally.
struct TileWalk {
    const uint16_t* kbase;   // this (stream, head)'s K pool / V pool / specials
    const uint16_t* vbase;
    const uint16_t* kspb;
    const uint16_t* vspb;
    const int* vis;
    int tpp, P, vis_n, vis_sp, slot_cap, sp_cap, pool_stride_k, pool_stride_v;
    int pi, ti;              // current page index and tile within it (pi == vis_n: specials)

    __device__ void seek(int t) {
        const int npt = vis_n * tpp;
        if (t < npt) {
            pi = t / tpp;
            ti = t - pi * tpp;
        } else {
            pi = vis_n;
            ti = t - npt;
        }
    }
    __device__ void next() {
        ++ti;
        if (pi < vis_n && ti == tpp) {
            ++pi;
            ti = 0;
        }
    }
    // K tile: 64 rows of 64; V^T tile: 64 rows of 64 positions at stride vstride.
    __device__ void get(const uint16_t*& k, const uint16_t*& v, int& vstride, int& len) const {
        const int off = ti * kTile;
        if (pi < vis_n) {
            const int page = __builtin_amdgcn_readfirstlane(vis[pi]);   // uniform
            k = kbase + (size_t)page * pool_stride_k + (size_t)off * kHeadDim;
            v = vbase + (size_t)page * pool_stride_v + off;
            vstride = slot_cap;
            len = min(kTile, P - off);
        } else {
            k = kspb + (size_t)off * kHeadDim;
            v = vspb + off;
            vstride = sp_cap;
            len = min(kTile, vis_sp - off);
        }
    }
};

__global__ __launch_bounds__(256) void k_attend_bf16(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kTile * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kHeadDim * kLds];
    __shared__ int s_vis[kMaxPool];

    // Logical workgroup id: consecutive physical ids go round-robin to the 8
    // XCDs, so the remap gives each XCD a contiguous range of logical ids; the
    // q-tiles of one (stream, head, split) share their K/V tiles in that XCD's L2.
    const int per_xcd = gridDim.x / 8;
    const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (L >= a.n_logical) return;
    const int qt = L % a.q_tiles;
    int rest = L / a.q_tiles;
    const int split = rest % a.splits;
    rest /= a.splits;
    const int h = rest % a.H;
    const int s = rest / a.H;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, col = lane & 31;
    const CacheState* st = a.states + s;
    TileWalk w;
    w.vis_n = st->vis_n;
    w.vis_sp = st->vis_sp_tokens;
    for (int i = tid; i < w.vis_n; i += 256) s_vis[i] = st->vis[i];
    w.vis = s_vis;
    w.tpp = a.tpp;
    w.P = a.P;
    w.slot_cap = a.slot_cap;
    w.sp_cap = a.sp_cap;
    w.pool_stride_k = a.slot_cap * kHeadDim;
    w.pool_stride_v = kHeadDim * a.slot_cap;
    w.kbase = (const uint16_t*)a.kpool + s * a.kpool_elems + (size_t)h * a.pool * a.slot_cap * kHeadDim;
    w.vbase = (const uint16_t*)a.vpool + s * a.kpool_elems + (size_t)h * a.pool * a.slot_cap * kHeadDim;
    w.kspb = (const uint16_t*)a.ksp + s * a.ksp_elems + (size_t)h * a.sp_cap * kHeadDim;
    w.vspb = (const uint16_t*)a.vsp + s * a.ksp_elems + (size_t)h * kHeadDim * a.sp_cap;

    const int n_tiles = w.vis_n * a.tpp + (w.vis_sp + kTile - 1) / kTile;
    const int t0 = (int)((long long)split * n_tiles / a.splits);
    const int t1 = (int)((long long)(split + 1) * n_tiles / a.splits);

    // Q^T operands of this wave's 32 queries (B operand: column = query),
    // pre-multiplied by c = log2(e)/sqrt(D) and rounded once to bf16, so the
    // matrix cores produce scores in base-2 exponent units.
    const float c = a.scale_log2;
    const int q = qt * kQB + wave * kQW + col;
    const bool qvalid = q < a.N;
    bf16x8 qf[4];
    {
        const uint16_t* qp = (const uint16_t*)a.q + (((size_t)s * a.N + (qvalid ? q : 0)) * a.H + h) * kHeadDim;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
            const uint4 u = qvalid ? *(const uint4*)(qp + dc * 16 + 8 * hh) : make_uint4(0, 0, 0, 0);
            const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qf[dc][2 * i] = (__bf16)(__uint_as_float(wv[i] << 16) * c);
                qf[dc][2 * i + 1] = (__bf16)(__uint_as_float(wv[i] & 0xFFFF0000u) * c);
            }
        }
    }

    f32x16 o0, o1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        o0[i] = 0.f;
        o1[i] = 0.f;
    }
    // Reference exponent M (shared by the two lanes of a query): the score
    // accumulators start at -M, so an MFMA result t is already c*q.k - M and
    // p = exp2(t).  M moves only when some t exceeds 8 (every p stays below
    // 2^8); the first tile sets it to the tile maximum.
    float M = 0.f, l = 0.f;
    f32x16 negM;
#pragma unroll
    for (int i = 0; i < 16; ++i) negM[i] = 0.f;
    bool first = true;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // staging: thread tid moves K rows (tid>>3) and (tid>>3)+32, chunk tid&7,
    // and the same rows of the V^T tile.
    const int srow = tid >> 3, schunk = (tid & 7) * 8;
    uint4 k0r, k1r, v0r, v1r;
    int len_next = 0;

    __syncthreads();   // s_vis ready
    if (t0 < t1) {
        w.seek(t0);
        const uint16_t *kp, *vp;
        int vs;
        w.get(kp, vp, vs, len_next);
        k0r = *(const uint4*)(kp + srow * kHeadDim + schunk);
        k1r = *(const uint4*)(kp + (srow + 32) * kHeadDim + schunk);
        v0r = *(const uint4*)(vp + (size_t)srow * vs + schunk);
        v1r = *(const uint4*)(vp + (size_t)(srow + 32) * vs + schunk);
    }
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        uint16_t* kt = lds_k[buf];
        uint16_t* vt = lds_v[buf];
        *(uint4*)&kt[srow * kLds + schunk] = k0r;
        *(uint4*)&kt[(srow + 32) * kLds + schunk] = k1r;
        *(uint4*)&vt[srow * kLds + schunk] = v0r;
        *(uint4*)&vt[(srow + 32) * kLds + schunk] = v1r;
        const int len = len_next;
        __syncthreads();
        if (t + 1 < t1) {
            w.next();
            const uint16_t *kp, *vp;
            int vs;
            w.get(kp, vp, vs, len_next);
            k0r = *(const uint4*)(kp + srow * kHeadDim + schunk);
            k1r = *(const uint4*)(kp + (srow + 32) * kHeadDim + schunk);
            v0r = *(const uint4*)(vp + (size_t)srow * vs + schunk);
            v1r = *(const uint4*)(vp + (size_t)(srow + 32) * vs + schunk);
        }

        // S^T = K Q^T - M for the tile's 64 keys: two 32-key blocks.  All
        // eight K fragments are read first so the LDS latency overlaps.
        bf16x8 ka[8];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
            ka[dc] = *(const bf16x8*)&kt[col * kLds + dc * 16 + 8 * hh];
            ka[4 + dc] = *(const bf16x8*)&kt[(32 + col) * kLds + dc * 16 + 8 * hh];
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the eight reads ahead of the products
        f32x16 s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], negM, 0, 0, 0);
        f32x16 s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[4], qf[0], negM, 0, 0, 0);
#pragma unroll
        for (int dc = 1; dc < 4; ++dc) {
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[4 + dc], qf[dc], s1, 0, 0, 0);
        }
        // V fragments for the second product, read while the scores finish.
        bf16x8 va[8];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            va[kc] = *(const bf16x8*)&vt[col * kLds + kc * 16 + 8 * hh];
            va[4 + kc] = *(const bf16x8*)&vt[(32 + col) * kLds + kc * 16 + 8 * hh];
        }
        // Key of s_kb[r]: kb*32 + 8*(r/4) + 4*hh + r%4.
        if (len < kTile) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
                if (key >= len) s0[r] = -INFINITY;
                if (32 + key >= len) s1[r] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(s0[0], s1[0]), s0[1]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s1[r]), s0[r + 1 < 16 ? r + 1 : 15]);
        if (first || __any(mx > 8.f)) {
            // rare: move M (jointly for both lanes of a query), never down
            // after the first tile, and rescale what was accumulated.
            const float d = fmaxf(mx, __shfl_xor(mx, 32));
            const float shift = first ? d : fmaxf(d, 0.f);
            first = false;
            M += shift;
            const float alpha = __builtin_amdgcn_exp2f(-shift);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                o0[i] *= alpha;
                o1[i] *= alpha;
                s0[i] -= shift;
                s1[i] -= shift;
                negM[i] = -M;
            }
        }
        bf16x8 pb[4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            pb[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(s0[r]);
            pb[2 + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(s1[r]);
        }
        // Row sum of the bf16 weights actually used in the product.
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pr = {pb[kc][2 * e], pb[kc][2 * e + 1]};
                l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
            }
        // O^T += V^T P^T.
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kc], pb[kc], o0, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[4 + kc], pb[kc], o1, 0, 0, 0);
        }
    }

    // Row sum over both half-waves; output O = O^T / l.
    l += __shfl_xor(l, 32);
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse_v = empty ? -INFINITY : (M + __log2f(l)) * 0.69314718055994531f;
    if (!qvalid) return;
    if (a.splits == 1) {
        uint16_t* op = (uint16_t*)a.out + (((size_t)s * a.N + q) * a.H + h) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hh;
                const f32x16& o = db ? o1 : o0;
                uint32_t wv[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const __bf16 lo = (__bf16)(o[4 * g + 2 * e] * inv);
                    const __bf16 hi = (__bf16)(o[4 * g + 2 * e + 1] * inv);
                    wv[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *(uint2*)(op + d0) = make_uint2(wv[0], wv[1]);
            }
        if (a.lse && hh == 0) a.lse[((size_t)s * a.H + h) * a.N + q] = lse_v;
    } else {
        const size_t row = (((size_t)s * a.H + h) * a.splits + split) * a.N + q;
        float* op = a.part_o + row * kHeadDim;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hh;
                const f32x16& o = db ? o1 : o0;
                *(float4*)(op + d0) = make_float4(o[4 * g] * inv, o[4 * g + 1] * inv,
                                                  o[4 * g + 2] * inv, o[4 * g + 3] * inv);
            }
        if (hh == 0) a.part_lse[row] = lse_v;
    }
}

// Merge of the key-range splits: out = sum_i w_i O_i / sum_i w_i with
// w_i = exp(lse_i - max lse); lse = max + log(sum w).  One thread per
// (stream, head, query, 4 channels).
template <typename T>
__global__ __launch_bounds__(256) void k_attend_combine(AttnArgs a) {
    const size_t idx = blockIdx.x * (size_t)256 + threadIdx.x;
    const size_t total = (size_t)a.S * a.H * a.N * 16;
    if (idx >= total) return;
    const int d4 = idx & 15;
    const size_t rest = idx >> 4;
    const int q = rest % a.N;
    const int sh = rest / a.N;   // s*H + h
    const int s = sh / a.H, h = sh % a.H;
    const size_t base = (size_t)sh * a.splits * a.N + q;
    float mx = -INFINITY;
    for (int i = 0; i < a.splits; ++i) mx = fmaxf(mx, a.part_lse[base + (size_t)i * a.N]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
    if (mx > -INFINITY) {
        for (int i = 0; i < a.splits; ++i) {
            const size_t row = base + (size_t)i * a.N;
            const float w = __expf(a.part_lse[row] - mx);
            const float4 o = *(const float4*)(a.part_o + row * kHeadDim + d4 * 4);
            acc[0] += w * o.x;
            acc[1] += w * o.y;
            acc[2] += w * o.z;
            acc[3] += w * o.w;
            wsum += w;
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    T* op = (T*)a.out + (((size_t)s * a.N + q) * a.H + h) * kHeadDim + d4 * 4;
    if constexpr (sizeof(T) == 2) {
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const __bf16 lo = (__bf16)(acc[2 * e] * inv);
            const __bf16 hi = (__bf16)(acc[2 * e + 1] * inv);
            w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *(uint2*)op = make_uint2(w[0], w[1]);
    } else {
        *(float4*)op = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
    if (d4 == 0 && a.lse) a.lse[(size_t)sh * a.N + q] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

// fp32: one query per thread, fp32 throughout (precise exp/log).
__global__ __launch_bounds__(64) void k_attend_f32(AttnArgs a) {
    __shared__ float ks[kTile][kHeadDim + 1];
    __shared__ float vs[kHeadDim][kTile + 1];
    const int h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
    const int q = blockIdx.x * 64 + tid;
    const bool qvalid = q < a.N;
    const CacheState* st = a.states + s;
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
        tile_ref<float>(a, s, h, t, n_patch_tiles, st->vis, vis_sp, kp, vp, vstride, len);
        __syncthreads();
        for (int i = tid; i < kTile * kHeadDim; i += 64) {
            const int r = i / kHeadDim, d = i % kHeadDim;
            ks[r][d] = kp[(size_t)r * kHeadDim + d];
            const int vr = i / kTile, vc = i % kTile;
            vs[vr][vc] = vp[(size_t)vr * vstride + vc];
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
    const int phys = (a.n_logical + 7) / 8 * 8;
    hipLaunchKernelGGL(k_attend_bf16, dim3(phys), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const size_t total = (size_t)a.S * a.H * a.N * 16;
    hipLaunchKernelGGL(k_attend_combine<uint16_t>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace rpkv
