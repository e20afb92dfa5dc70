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
//  * tiles stream from HBM straight into LDS (buffer_load ... lds: no staging
//    registers, the page offset in a scalar register) through rings of 2 K
//    and 3 V^T stages, one barrier per tile; 16-byte chunks are XOR-swizzled
//    so operand reads hit 64 distinct banks (40 KB of LDS per workgroup);
//  * scores are formed transposed, S^T = K Q^T (keys on the MFMA rows, queries
//    on the columns): each lane holds 16 scores of one query per 32-key half
//    tile, so the softmax statistics stay in-lane but for one exchange with
//    the lane 32 apart; P^T rounded to bf16 is directly the B operand of
//    O^T = V^T P^T, V being stored transposed in the cache in the key order
//    this layout produces;
//  * the wave is software-pipelined by half tiles: the score products of the
//    next half are issued before the exponentials of the current one, so the
//    matrix core and the vector ALU work side by side (the next half of the
//    last half tile of tile i is the first half of tile i+1, formed after the
//    barrier of tile i+1);
//  * scores s = q.k come out of the matrix core in fp32 from the stored bf16
//    Q and K (no extra rounding of Q); one fused multiply-add per score turns
//    s into the base-2 exponent t = s*log2(e)/sqrt(D) - M (M: the running
//    reference max), and p = exp2(t) costs one transcendental; M moves (and
//    the accumulated output is rescaled) only when a score exceeds it by 2^8;
//  * several splits of the key range are merged by their log-sum-exp.
#include "rpkv_internal.h"

namespace rpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kWaves = 4;
constexpr int kQW = 32;                          // queries per wave
constexpr int kQB = kWaves * kQW;                // queries per workgroup
constexpr int kTileBytes = kTile * kHeadDim * 2; // one 64x64 bf16 tile: 8 KB
constexpr int kHalfBytes = 32 * 128;             // 32 rows of a tile
// LDS rings: K tiles in 2 stages, V^T tiles in 3.  K of tile i is read from
// the barrier of tile i up to the barrier of tile i+1, V^T of tile i up to
// the barrier of tile i+2; tile i+2 is loaded from the barrier of tile i+1.
constexpr int kKStages = 2, kVStages = 3;
constexpr int kGroup = 6;                        // tiles per unrolled group (lcm of the rings)
constexpr int kLdsBytes = (kKStages + kVStages) * kTileBytes;
// Word 3 of a raw (unstructured) buffer resource on gfx9: 32-bit data format.
constexpr int kBufWord3 = 0x00020000;

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Raw buffer resource over [p, p + bytes), built from scalar registers.
__device__ inline __amdgpu_buffer_rsrc_t buffer_over(const char* p, size_t bytes) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)uniform((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)uniform((int)(uint32_t)(v >> 32));
    const int n = uniform((int)(uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, kBufWord3);
}

// Loads of one (stream, head): buffer resources over its K pool, V^T pool and
// special K / V^T, and this lane's byte offsets inside the 8-row slabs it
// loads (its row, and the 16-byte chunk that belongs at its slot under the
// swizzle).  All page arithmetic is scalar.
struct Loader {
    __amdgpu_buffer_rsrc_t kpool, vpool, ksp, vsp;
    const int* vis;          // visible pages (read through the scalar cache)
    int vis_n, tpp, slot_cap;
    uint32_t lk0, lk1, lvp0, lvp1, lvs0, lvs1;

    // Issues this wave's share of tile t (rows 16*wave .. 16*wave+15 of the K
    // tile and of the V^T tile, 8 rows per instruction) into an LDS stage.
    __device__ void issue(int t, char* kstage, char* vstage, int wave) const {
        char* k0 = kstage + wave * 2 * 8 * 128;
        char* v0 = vstage + wave * 2 * 8 * 128;
        const int npt = vis_n * tpp;
        if (t < npt) {
            const int pi = t / tpp;
            const uint32_t off = (uint32_t)(t - pi * tpp) * kTile;
            const uint32_t page = (uint32_t)uniform(vis[pi]);
            const uint32_t ko = (page * (uint32_t)slot_cap + off) * 128u;
            const uint32_t vo = page * (uint32_t)slot_cap * 128u + off * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kpool, (lds_void_ptr)k0, 16, lk0, ko, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kpool, (lds_void_ptr)(k0 + 1024), 16, lk1, ko, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vpool, (lds_void_ptr)v0, 16, lvp0, vo, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vpool, (lds_void_ptr)(v0 + 1024), 16, lvp1, vo, 0, 0);
        } else {
            const uint32_t off = (uint32_t)(t - npt) * kTile;
            const uint32_t ko = off * 128u, vo = off * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ksp, (lds_void_ptr)k0, 16, lk0, ko, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ksp, (lds_void_ptr)(k0 + 1024), 16, lk1, ko, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vsp, (lds_void_ptr)v0, 16, lvs0, vo, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vsp, (lds_void_ptr)(v0 + 1024), 16, lvs1, vo, 0, 0);
        }
    }
};

// Running state of one wave's 32 queries.
struct Acc {
    f32x16 o0, o1;     // O^T, d rows 0-31 and 32-63
    float lp[4];       // partial row sums
    float M;           // reference max of the base-2 exponents
    float c;           // log2(e)/sqrt(D)
    bool first;
};

// s = q.k for the 32 keys of half kb of a tile (rows 32*kb + col of the K
// tile; chunk 2*j + hh is k-step j).
__device__ __forceinline__ f32x16 scores(const char* tile, int kb, const int* foff, const bf16x8* qf) {
    const char* t = tile + kb * kHalfBytes;
    const bf16x8 k0 = *(const bf16x8*)(t + foff[0]);
    const bf16x8 k1 = *(const bf16x8*)(t + foff[1]);
    const bf16x8 k2 = *(const bf16x8*)(t + foff[2]);
    const bf16x8 k3 = *(const bf16x8*)(t + foff[3]);
    const f32x16 zero = {};
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[0], zero, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[1], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k2, qf[2], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k3, qf[3], s, 0, 0, 0);
    return s;
}

// One half tile: the softmax weights of sc (half kb of `tile`, len valid keys
// in the tile), their output products, and -- interleaved with them, so the
// matrix core works while the exponentials run -- the scores of the next half
// tile into nxt (K rows at knext; the caller makes sure they are loaded, or
// ignores nxt).  Key of sc[r]: 32*kb + 8*(r/4) + 4*hh + r%4; its V^T column
// sits at that key's slot, chunk 4*kb + 2*(r/8) + hh.
__device__ __forceinline__ void step(f32x16& sc, f32x16& nxt, const char* vt, int kb, int len,
                                     const char* knext, const int* foff, const bf16x8* qf, int hh,
                                     Acc& A) {
    if (len < 32 * kb + 32) {   // ragged: keys past the tile's end do not count
        const int lim = len - 32 * kb - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
    }
    const float ma = max3f(sc[0], sc[1], sc[2]);
    const float mb = max3f(sc[3], sc[4], sc[5]);
    const float mc = max3f(sc[6], sc[7], sc[8]);
    const float md = max3f(sc[9], sc[10], sc[11]);
    const float me = max3f(sc[12], sc[13], sc[14]);
    const float mx = max3f(max3f(ma, mb, mc), fmaxf(md, me), sc[15]);
    // (A half with no valid key -- a tile past a short page's tokens -- has
    // every score at -inf: it moves nothing and adds nothing.)
    if ((A.first && __any(mx > -INFINITY)) || __any(fmaf(mx, A.c, -A.M) > 8.f)) {
        // rare: move M (jointly for both lanes of a query; never down after
        // the first half tile) and rescale what was accumulated.
        const float d = fmaxf(mx, __shfl_xor(mx, 32)) * A.c;
        const float m_new = A.first ? d : fmaxf(d, A.M);
        const float alpha = A.first ? 0.f : __builtin_amdgcn_exp2f(A.M - m_new);
        A.first = false;
        A.M = m_new;
#pragma unroll
        for (int e = 0; e < 4; ++e) A.lp[e] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            A.o0[r] *= alpha;
            A.o1[r] *= alpha;
        }
    }
    // LDS operands: V^T fragments of this half, K fragments of the next.
    bf16x8 v[2][2], k[4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        v[m][0] = *(const bf16x8*)(vt + foff[2 * kb + m]);
        v[m][1] = *(const bf16x8*)(vt + kHalfBytes + foff[2 * kb + m]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = *(const bf16x8*)(knext + foff[j]);
    // p = exp2(t), rounded to bf16 in pairs for the products; the row sums
    // add the fp32 weights (plain adds: the bf16 dot instruction would hold
    // up the matrix core).
    bf16x2 pr[8];
    const f32x16 zero = {};
    const float nm = -A.M;
#define RPKV_EXP_PAIR(e)                                                                           \
    do {                                                                                           \
        const f32x2 x_ = {__builtin_amdgcn_exp2f(fmaf(sc[2 * (e)], A.c, nm)),                      \
                          __builtin_amdgcn_exp2f(fmaf(sc[2 * (e) + 1], A.c, nm))};                 \
        pr[e] = __builtin_convertvector(x_, bf16x2);                                               \
        A.lp[(e) & 3] += x_[0] + x_[1];                                                            \
    } while (0)
    nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[0], qf[0], zero, 0, 0, 0);
    RPKV_EXP_PAIR(0);
    RPKV_EXP_PAIR(1);
    nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[1], qf[1], nxt, 0, 0, 0);
    RPKV_EXP_PAIR(2);
    RPKV_EXP_PAIR(3);
    const bf16x8 pb0 = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                               __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
    nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[2], qf[2], nxt, 0, 0, 0);
    A.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[0][0], pb0, A.o0, 0, 0, 0);
    RPKV_EXP_PAIR(4);
    RPKV_EXP_PAIR(5);
    nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[3], qf[3], nxt, 0, 0, 0);
    A.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[0][1], pb0, A.o1, 0, 0, 0);
    RPKV_EXP_PAIR(6);
    RPKV_EXP_PAIR(7);
#undef RPKV_EXP_PAIR
    const bf16x8 pb1 = __builtin_shufflevector(__builtin_shufflevector(pr[4], pr[5], 0, 1, 2, 3),
                                               __builtin_shufflevector(pr[6], pr[7], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
    A.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[1][0], pb1, A.o0, 0, 0, 0);
    A.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[1][1], pb1, A.o1, 0, 0, 0);
    // Keep this half's row sums here (not sunk past the barrier that may
    // follow), so its weights die now.
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(A.lp[e]));
    __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(256) void k_attend_bf16(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
    __shared__ int s_vlen[kMaxPool];   // tokens of each visible patch page
    char* const kring = lds;
    char* const vring = lds + kKStages * kTileBytes;

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

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int hh = lane >> 5, col = lane & 31;
    const CacheState* st = a.states + s;
    // The frame's own tokens are the queries: a q-tile wholly past them has
    // nothing to do.
    const int n_q = uniform(st->n_query);
    if (qt * kQB >= n_q) return;
    const int vis_n = uniform(st->vis_n);
    const int vis_sp = uniform(st->vis_sp_tokens);

    Loader ld;
    {
        const size_t head_bytes = (size_t)a.pool * a.slot_cap * kHeadDim * 2;
        const size_t sp_bytes = (size_t)a.sp_cap * kHeadDim * 2;
        const char* kp = a.kpool + (s * a.kpool_elems) * 2 + h * head_bytes;
        const char* vp = a.vpool + (s * a.kpool_elems) * 2 + h * head_bytes;
        const char* ks = a.ksp + (s * a.ksp_elems) * 2 + h * sp_bytes;
        const char* vs = a.vsp + (s * a.ksp_elems) * 2 + h * sp_bytes;
        ld.kpool = buffer_over(kp, head_bytes);
        ld.vpool = buffer_over(vp, head_bytes);
        ld.ksp = buffer_over(ks, sp_bytes);
        ld.vsp = buffer_over(vs, sp_bytes);
    }
    ld.vis = st->vis;
    ld.vis_n = vis_n;
    ld.tpp = a.tpp;
    ld.slot_cap = a.slot_cap;
    // LDS tile layout: row r at r*128 bytes, its 16-byte chunk c stored at
    // position c ^ ((r >> 1) & 7).  A 128-byte row spans half of the 64 LDS
    // banks, so any 16 consecutive rows read at one logical chunk (the 16 lanes
    // the LDS serves together) land on 16 distinct bank quads.
    // Per-lane load offsets (row = 16*wave + 8*slab + lane/8).
    {
        uint32_t lk[2], lvp[2], lvs[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (wave * 2 + i) * 8 + (lane >> 3);
            const int ch = (lane & 7) ^ ((r >> 1) & 7);
            lk[i] = r * 128 + ch * 16;
            lvp[i] = r * a.slot_cap * 2 + ch * 16;
            lvs[i] = r * a.sp_cap * 2 + ch * 16;
        }
        ld.lk0 = lk[0];
        ld.lk1 = lk[1];
        ld.lvp0 = lvp[0];
        ld.lvp1 = lvp[1];
        ld.lvs0 = lvs[0];
        ld.lvs1 = lvs[1];
    }
    const int n_patch_tiles = vis_n * a.tpp;
    const int n_tiles = n_patch_tiles + (vis_sp + kTile - 1) / kTile;
    const int t0 = uniform((int)((long long)split * n_tiles / a.splits));
    const int t1 = uniform((int)((long long)(split + 1) * n_tiles / a.splits));
    const int n = t1 - t0;

    // Q^T operands of this wave's 32 queries (B operand: column = query): the
    // stored bf16 values as they are.
    const int q = qt * kQB + wave * kQW + col;
    const bool qvalid = q < n_q;
    bf16x8 qf[4];
    {
        const uint16_t* qp = (const uint16_t*)a.q + (((size_t)s * a.N + (qvalid ? q : 0)) * a.H + h) * kHeadDim;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
            const uint4 u = qvalid ? *(const uint4*)(qp + dc * 16 + 8 * hh) : make_uint4(0, 0, 0, 0);
            qf[dc] = __builtin_bit_cast(bf16x8, u);
        }
    }

    Acc A;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        A.o0[i] = 0.f;
        A.o1[i] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) A.lp[e] = 0.f;
    A.M = 0.f;
    A.c = a.scale_log2;
    A.first = true;

    // Operand byte offsets inside a tile ((row >> 1) & 7 == (col >> 1) & 7 for
    // every 32-row block).
    int foff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) foff[j] = col * 128 + (((2 * j + hh) ^ ((col >> 1) & 7)) << 4);

    // Page lengths: all P when every visible page holds a whole grid (then
    // nothing is read per tile), else an LDS copy.
    const bool vis_full = uniform(st->vis_full) != 0;
    if (!vis_full)
        for (int i = tid; i < vis_n; i += 256) s_vlen[i] = st->vis_len[i];

    // Prologue: tiles 0 and 1 in flight; wait for tile 0 (the barrier also
    // publishes s_vlen).
    if (n > 0) ld.issue(t0, kring, vring, wave);
    if (n > 1) ld.issue(t0 + 1, kring + kTileBytes, vring + kTileBytes, wave);
    if (n > 1)
        wait_vmcnt<4>();
    else
        wait_vmcnt<0>();
    __syncthreads();

    // sA: first half of the tile being computed, sB: its second half.  The
    // products of a half are formed one half ahead of its softmax; past the
    // last tile they read a stale stage and are never used.
    // Valid keys of a tile: a patch page holds the tokens its frame had
    // (tiles past them have none), the special stream vis_sp.  Worked out
    // one tile ahead from a walk over (page, tile in page); the page length
    // is looked up once per page, and not at all when every page is whole.
    auto page_len = [&](int pi) { return vis_full ? a.P : uniform(s_vlen[pi]); };
    int wpi = t0 / a.tpp, wti = t0 % a.tpp;   // walk position: the next tile
    int wpl = wpi < vis_n ? page_len(wpi) : 0;
    auto walk_len = [&](int t) {
        return t < n_patch_tiles ? min(kTile, wpl - wti * kTile)
                                 : min(kTile, vis_sp - (t - n_patch_tiles) * kTile);
    };
    auto walk_next = [&]() {
        if (++wti == a.tpp) {
            wti = 0;
            ++wpi;
            if (wpi < vis_n) wpl = page_len(wpi);
        }
    };
    int len_next = walk_len(t0);
    f32x16 sA = scores(kring, 0, foff, qf);
    f32x16 sB;
    // Tiles in groups of kGroup, so every stage offset is a constant that
    // folds into the LDS instructions' immediate offsets.
    for (int i0 = 0; i0 < n; i0 += kGroup) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int i = i0 + u, t = t0 + i;
            if (i >= n) break;
            const char* kcur = kring + (u % kKStages) * kTileBytes;
            const char* knxt = kring + ((u + 1) % kKStages) * kTileBytes;
            const char* vcur = vring + (u % kVStages) * kTileBytes;
            const int len = len_next;
            walk_next();
            len_next = walk_len(t + 1);
            step(sA, sB, vcur, 0, len, kcur + kHalfBytes, foff, qf, hh, A);
            if (i + 1 < n) {
                // Tile i+1 landed for every wave, every wave is done with K of
                // tile i and V^T of tile i-1: their stages take tile i+2.
                wait_vmcnt<0>();
                __syncthreads();
                if (i + 2 < n)
                    ld.issue(t + 2, kring + ((u + 2) % kKStages) * kTileBytes,
                             vring + ((u + 2) % kVStages) * kTileBytes, wave);
            }
            if (len > 32)
                step(sB, sA, vcur, 1, len, knxt, foff, qf, hh, A);
            else
                sA = scores(knxt, 0, foff, qf);
        }
    }

    // Row sum over both half-waves; output O = O^T / l.
    float l = (A.lp[0] + A.lp[1]) + (A.lp[2] + A.lp[3]);
    l += __shfl_xor(l, 32);
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse_v = empty ? -INFINITY : (A.M + __log2f(l)) * 0.69314718055994531f;
    // Largest accumulator of the query (both half-waves hold 32 of its 64
    // channels): the split path scales its row by it.
    float mo = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) mo = max3f(mo, fabsf(A.o0[r]), fabsf(A.o1[r]));
    mo = fmaxf(mo, __shfl_xor(mo, 32));
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
        // Partial outputs in fp16 (RNE), each row scaled by the power of two
        // 2^-e that brings its largest accumulator into [1, 2) (e clamped to
        // [-126, 126]), so fp16 keeps 11 significant bits of every row
        // whatever the range of V: no overflow for large V, no subnormals for
        // small V.  The row's factor 2^e / l goes to the merge in fp32 beside
        // the LSE.  Scaling by a power of two is exact, so V scaled by 2^k
        // gives exactly the same fp16 words.
        const int b = min(max((int)(__float_as_uint(mo) >> 23), 1), 253);   // biased exponent
        const float down = __uint_as_float((uint32_t)(254 - b) << 23);      // 2^-e
        const float fac = inv * __uint_as_float((uint32_t)b << 23);         // 2^e / l
        uint16_t* op = a.part_o + row * kHeadDim;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hh;
                const f32x16& o = db ? A.o1 : A.o0;
                uint32_t wv[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const _Float16 lo = (_Float16)(o[4 * g + 2 * e] * down);
                    const _Float16 hi = (_Float16)(o[4 * g + 2 * e + 1] * down);
                    wv[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *(uint2*)(op + d0) = make_uint2(wv[0], wv[1]);
            }
        if (hh == 0) a.part_ls[row] = make_float2(lse_v, fac);
    }
}

hipError_t launch_attend_bf16_main(const AttnArgs& a, hipStream_t st) {
    const int phys = (a.n_logical + 7) / 8 * 8;   // a multiple of the 8 XCDs
    hipLaunchKernelGGL(k_attend_bf16, dim3(phys), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace rpkv
