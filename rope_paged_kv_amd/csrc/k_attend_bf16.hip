// Paged attention of one frame's tokens over the visible page table, bf16 on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// What is computed (page "How 3D RoPE Positional Encoding Works with the Paged
// KV Cache in LingBot-Map", section "Attention Computation with Cached RoPE";
// page "How LingBot-Map Achieves Real-Time 3D Reconstruction", section
// "Per-Frame Processing and Causal Attention"): for every query token of the
// frame and head, softmax(q . k / sqrt(D)) weighted sum of v over the visible
// keys -- the patch tokens of the visible patch pages and the tokens of the
// visible special pages.
//
// Structure:
//  * a workgroup of 4 waves takes 128 queries of one (stream, head) and one
//    split of the visible key range; each wave owns 32 queries;
//  * keys are walked in tiles of 64 that never straddle a page (a patch page
//    of P tokens is ceil(P/64) tiles; the special stream, whose pages are
//    appended in order and never evicted, is contiguous per head);
//  * tiles stream from HBM straight into LDS (global_load_lds_dwordx4: no
//    staging registers) through a 4-stage ring, two tiles ahead, one barrier
//    per tile; 16-byte chunks are XOR-swizzled so operand reads hit 64
//    distinct banks;
//  * scores are formed transposed, S^T = K Q^T (keys on the MFMA rows, queries
//    on the columns): each lane holds 32 scores of one query, so the softmax
//    statistics stay in-lane but for one exchange with the lane 32 apart;
//    P^T rounded to bf16 is directly the B operand of O^T = V^T P^T, V being
//    stored transposed in the cache in the key order this layout produces;
//  * each pair of output products follows the exponentials of its 16 keys,
//    so the matrix core works on one batch while the next is exponentiated;
//  * Q is pre-multiplied by log2(e)/sqrt(D) and the score accumulators start
//    at -M (the running reference max), so a product is already the base-2
//    exponent and p = exp2(t) costs one transcendental; M moves (and the
//    accumulated output is rescaled) only when a score exceeds it by 2^8;
//  * several splits of the key range are merged by their log-sum-exp.
#include "rpkv_internal.h"

namespace rpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kWaves = 4;
constexpr int kQW = 32;                          // queries per wave
constexpr int kQB = kWaves * kQW;                // queries per workgroup
constexpr int kStages = 4;
constexpr int kTileBytes = kTile * kHeadDim * 2; // one 64x64 bf16 tile: 8 KB
constexpr int kStageBytes = 2 * kTileBytes;      // K tile + V^T tile


// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Position in the tile sequence of a split: patch page index pi (pi == vis_n:
// the special stream) and tile ti within it.
struct Cursor {
    int pi, ti;
};

struct Walk {
    const uint16_t* kbase;   // this (stream, head): K pool, V^T pool, K / V^T specials
    const uint16_t* vbase;
    const uint16_t* kspb;
    const uint16_t* vspb;
    const int* vis;          // visible pages (LDS copy)
    int tpp, P, vis_n, vis_sp, slot_cap, sp_cap;

    __device__ Cursor at(int t) const {
        const int npt = vis_n * tpp;
        if (t < npt) return {t / tpp, t % tpp};
        return {vis_n, t - npt};
    }
    __device__ void next(Cursor& c) const {
        ++c.ti;
        if (c.pi < vis_n && c.ti == tpp) {
            ++c.pi;
            c.ti = 0;
        }
    }
    __device__ int len(const Cursor& c) const {
        return min(kTile, (c.pi < vis_n ? P : vis_sp) - c.ti * kTile);
    }
    // Issues this wave's share of the loads of tile c into an LDS stage: rows
    // 16*wave .. 16*wave+15 of the K tile and of the V^T tile, 8 rows per
    // instruction.  k0/k1 (v*0/v*1) are this lane's byte offsets inside the
    // two 8-row slabs: its row, and the 16-byte chunk that belongs at its slot
    // under the swizzle.
    __device__ void issue(const Cursor& c, char* stage, int wave, uint32_t k0, uint32_t k1,
                          uint32_t vpage0, uint32_t vpage1, uint32_t vsp0, uint32_t vsp1) const {
        const int off = c.ti * kTile;
        const char* kp;
        const char* vp;
        uint32_t v0, v1;
        if (c.pi < vis_n) {
            const int page = __builtin_amdgcn_readfirstlane(vis[c.pi]);
            kp = (const char*)(kbase + ((size_t)page * slot_cap + off) * kHeadDim);
            vp = (const char*)(vbase + (size_t)page * kHeadDim * slot_cap + off);
            v0 = vpage0;
            v1 = vpage1;
        } else {
            kp = (const char*)(kspb + (size_t)off * kHeadDim);
            vp = (const char*)(vspb + off);
            v0 = vsp0;
            v1 = vsp1;
        }
        char* s0 = stage + wave * 2 * 8 * 128;
        __builtin_amdgcn_global_load_lds(kp + k0, (lds_void_ptr)s0, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(kp + k1, (lds_void_ptr)(s0 + 8 * 128), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + v0, (lds_void_ptr)(s0 + kTileBytes), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + v1, (lds_void_ptr)(s0 + kTileBytes + 8 * 128), 16, 0, 0);
    }
};

// Reads the eight 16-byte operand fragments of one swizzled 64x64 tile that
// this lane needs (rows col and 32+col, chunks 2*j+hh).
__device__ inline void read_frags(const char* tile, const int* off, bf16x8* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[j] = *(const bf16x8*)(tile + off[j]);
        f[4 + j] = *(const bf16x8*)(tile + 32 * 128 + off[j]);
    }
}

// Running state of one wave's 32 queries.
struct Acc {
    f32x16 o0, o1;     // O^T, d rows 0-31 and 32-63
    f32x16 negM;       // -M in every element: the score accumulators' start
    float M, l;
    bool first;
};

// Everything one wave does for key tile i: wait for it, hand tile i+3 to the
// loader, form its scores, softmax, and the output product.
struct Ctx {
    const Walk* w;
    char* lds;
    const bf16x8* qf;
    const int* foff;
    int wave, hh, n;
    uint32_t lk0, lk1, lvp0, lvp1, lvs0, lvs1;
};

__device__ __forceinline__ void step(const Ctx& x, int i, Cursor& ld, Cursor& cp, Acc& A) {
    // Tile i landed for every wave (tiles i+1, i+2 may still be in flight), and
    // every wave is done with tile i-1, whose stage now takes tile i+3.
    if (i + 2 < x.n)
        wait_vmcnt<8>();
    else if (i + 1 < x.n)
        wait_vmcnt<4>();
    else
        wait_vmcnt<0>();
    __syncthreads();
    if (i + kStages - 1 < x.n) {
        x.w->issue(ld, x.lds + ((i + kStages - 1) % kStages) * kStageBytes, x.wave, x.lk0, x.lk1,
                   x.lvp0, x.lvp1, x.lvs0, x.lvs1);
        x.w->next(ld);
    }
    const int len = x.w->len(cp);
    x.w->next(cp);
    const char* cur = x.lds + (i % kStages) * kStageBytes;

    // Scores t = c*q.k - M of the tile's 64 keys (two 32-key blocks).
    bf16x8 frag[8];
    read_frags(cur, x.foff, frag);
    f32x16 sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[0], x.qf[0], A.negM, 0, 0, 0);
    f32x16 sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[4], x.qf[0], A.negM, 0, 0, 0);
#pragma unroll
    for (int j = 1; j < 4; ++j) {
        sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[j], x.qf[j], sc0, 0, 0, 0);
        sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[4 + j], x.qf[j], sc1, 0, 0, 0);
    }
    // V^T fragments, read while the scores finish.
    read_frags(cur + kTileBytes, x.foff, frag);

    // Ragged tile: keys past its end do not count.  Key of sc_kb[r]:
    // kb*32 + 8*(r/4) + 4*hh + r%4.
    if (len < kTile) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * x.hh + (r & 3);
            if (key >= len) sc0[r] = -INFINITY;
            if (32 + key >= len) sc1[r] = -INFINITY;
        }
    }
    // Four independent max chains over 8 scores each, then combined.
    float m4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x16& sc = g < 2 ? sc0 : sc1;
        const int r0 = (g & 1) * 8;
        float m = max3f(sc[r0], sc[r0 + 1], sc[r0 + 2]);
        m = max3f(m, sc[r0 + 3], sc[r0 + 4]);
        m = max3f(m, sc[r0 + 5], sc[r0 + 6]);
        m4[g] = fmaxf(m, sc[r0 + 7]);
    }
    const float mx = max3f(m4[0], m4[1], fmaxf(m4[2], m4[3]));
    if (A.first || __any(mx > 8.f)) {
        // rare: move M (jointly for both lanes of a query; never down after
        // the first tile) and rescale what was accumulated.
        const float d = fmaxf(mx, __shfl_xor(mx, 32));
        const float shift = A.first ? d : fmaxf(d, 0.f);
        A.first = false;
        A.M += shift;
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        A.l *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            A.o0[r] *= alpha;
            A.o1[r] *= alpha;
            sc0[r] -= shift;
            sc1[r] -= shift;
            A.negM[r] = -A.M;
        }
    }

    // Weights p = exp2(t) of 16 keys at a time, each batch followed by its
    // two output products; the row sum (four independent partial sums) uses
    // the bf16 weights the products use.
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float lp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        const f32x16& sc = kc < 2 ? sc0 : sc1;
        const int r0 = (kc & 1) * 8;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)__builtin_amdgcn_exp2f(sc[r0 + e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2 pr = {pb[2 * e], pb[2 * e + 1]};
            lp[e] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lp[e], false);
        }
        A.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[kc], pb, A.o0, 0, 0, 0);
        A.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[4 + kc], pb, A.o1, 0, 0, 0);
    }
    A.l += (lp[0] + lp[1]) + (lp[2] + lp[3]);
}

__global__ __launch_bounds__(256) void k_attend_bf16(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];
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
    Walk w;
    w.vis_n = st->vis_n;
    w.vis_sp = st->vis_sp_tokens;
    for (int i = tid; i < w.vis_n; i += 256) s_vis[i] = st->vis[i];
    w.vis = s_vis;
    w.tpp = a.tpp;
    w.P = a.P;
    w.slot_cap = a.slot_cap;
    w.sp_cap = a.sp_cap;
    const size_t head_pool = (size_t)h * a.pool * a.slot_cap * kHeadDim;
    w.kbase = (const uint16_t*)a.kpool + s * a.kpool_elems + head_pool;
    w.vbase = (const uint16_t*)a.vpool + s * a.kpool_elems + head_pool;
    w.kspb = (const uint16_t*)a.ksp + s * a.ksp_elems + (size_t)h * a.sp_cap * kHeadDim;
    w.vspb = (const uint16_t*)a.vsp + s * a.ksp_elems + (size_t)h * kHeadDim * a.sp_cap;

    const int n_tiles = w.vis_n * a.tpp + (w.vis_sp + kTile - 1) / kTile;
    const int t0 = (int)((long long)split * n_tiles / a.splits);
    const int t1 = (int)((long long)(split + 1) * n_tiles / a.splits);
    const int n = t1 - t0;

    // Q^T operands of this wave's 32 queries (B operand: column = query),
    // pre-multiplied by c = log2(e)/sqrt(D) and rounded once to bf16.
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

    Acc A;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        A.o0[i] = 0.f;
        A.o1[i] = 0.f;
        A.negM[i] = 0.f;
    }
    A.M = 0.f;
    A.l = 0.f;
    A.first = true;

    // LDS tile layout: row r at r*128 bytes, its 16-byte chunk c stored at
    // position c ^ ((r >> 1) & 7).  A 128-byte row spans half of the 64 LDS
    // banks, so any 16 consecutive rows read at one logical chunk (the 16 lanes
    // the LDS serves together) land on 16 distinct bank quads.
    // Per-lane load offsets (row = 16*wave + 8*slab + lane/8).
    uint32_t lk[2], lvp[2], lvs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = (wave * 2 + i) * 8 + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        lk[i] = (r * kHeadDim + ch * 8) * 2;
        lvp[i] = (r * a.slot_cap + ch * 8) * 2;
        lvs[i] = (r * a.sp_cap + ch * 8) * 2;
    }
    // Operand byte offsets inside a tile ((row >> 1) & 7 == (col >> 1) & 7 for
    // both 32-row blocks).
    int foff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) foff[j] = col * 128 + (((2 * j + hh) ^ ((col >> 1) & 7)) << 4);

    __syncthreads();   // s_vis ready

    // Prologue: tiles 0 .. kStages-2 in flight.
    Cursor ld = w.at(t0), cp = ld;
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
        if (i < n) {
            w.issue(ld, lds + i * kStageBytes, wave, lk[0], lk[1], lvp[0], lvp[1], lvs[0], lvs[1]);
            w.next(ld);
        }
    Ctx x;
    x.w = &w;
    x.lds = lds;
    x.qf = qf;
    x.foff = foff;
    x.wave = wave;
    x.hh = hh;
    x.n = n;
    x.lk0 = lk[0];
    x.lk1 = lk[1];
    x.lvp0 = lvp[0];
    x.lvp1 = lvp[1];
    x.lvs0 = lvs[0];
    x.lvs1 = lvs[1];
    for (int i = 0; i < n; ++i) step(x, i, ld, cp, A);

    // Row sum over both half-waves; output O = O^T / l.
    float l = A.l + __shfl_xor(A.l, 32);
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse_v = empty ? -INFINITY : (A.M + __log2f(l)) * 0.69314718055994531f;
    if (!qvalid) return;
    if (a.splits == 1) {
        uint16_t* op = (uint16_t*)a.out + (((size_t)s * a.N + q) * a.H + h) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hh;
                const f32x16& o = db ? A.o1 : A.o0;
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
                const f32x16& o = db ? A.o1 : A.o0;
                *(float4*)(op + d0) = make_float4(o[4 * g] * inv, o[4 * g + 1] * inv,
                                                  o[4 * g + 2] * inv, o[4 * g + 3] * inv);
            }
        if (hh == 0) a.part_lse[row] = lse_v;
    }
}

hipError_t launch_attend_bf16_main(const AttnArgs& a, hipStream_t st) {
    const int phys = (a.n_logical + 7) / 8 * 8;   // a multiple of the 8 XCDs
    hipLaunchKernelGGL(k_attend_bf16, dim3(phys), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace rpkv
