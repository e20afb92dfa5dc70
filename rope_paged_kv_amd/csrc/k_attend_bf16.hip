// Paged attention of one frame's tokens over the visible page table, bf16 on
// the gfx950 matrix cores, fp32 accumulation.
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
//    appended in order and never evicted, is contiguous per head), each tile
//    in two halves of 32 keys;
//  * tiles stream from HBM straight into LDS (buffer_load ... lds: no staging
//    registers, the page offset in a scalar register) through rings of 3 K
//    and 3 V^T stages, each load issued two tiles before its use and waited
//    for with a counted wait, one barrier per tile; 16-byte chunks are
//    XOR-swizzled so operand reads hit 64 distinct banks;
//  * scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16:
//    keys on the rows, queries on the columns): each lane holds 16 scores of
//    one query per half tile; P^T rounded to bf16 is directly the B operand of
//    O^T = V^T P^T, V being stored transposed in the cache in the key order
//    this layout produces;
//  * software pipeline over half tiles: the step of half h issues the scores
//    of half h+1 and the output products of half h-1 on the matrix core, and
//    the softmax of half h on the vector ALU -- nothing in a step waits for
//    another part of the same step, so the waves of a SIMD overlap one's
//    matrix work with another's vector work;
//  * the row sums l = sum p are formed on the matrix core too, from the same
//    bf16 P^T operand (v_mfma_f32_16x16x32_bf16 against a 0/1 selection
//    matrix, so numerator and denominator use the same rounded weights);
//  * one fused multiply-add per score gives the base-2 exponent
//    t = s*log2(e)/sqrt(D) - M from the fp32 score of the stored bf16 Q and K
//    (no extra rounding of Q), and p = exp2(t); M sits 7 above the running
//    max, so weights stay below 2^-7, and moves only when some weight reaches
//    2, i.e. a score beats that max by 2^8 (checked on the packed bf16
//    weights with a few bit operations instead of a max per score); the
//    accumulated outputs and row sums are rescaled then;
//  * several splits of the key range are merged by their log-sum-exp.
#include "rpkv_internal.h"

namespace rpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
// Read-only during the kernel and read with uniform indices: loads through
// this pointer go to the scalar cache (s_load), which leaves the vector
// memory counter -- the one the tile loads are waited on with -- alone.
typedef const int __attribute__((address_space(4)))* cint_ptr;

constexpr int kWaves = 4;
constexpr int kQW = 32;                          // queries per wave
constexpr int kQB = kWaves * kQW;                // queries per workgroup
constexpr int kTileBytes = kTile * kHeadDim * 2; // one 64x64 bf16 tile: 8 KB
constexpr int kHalfBytes = 32 * 128;             // 32 rows of a tile
// LDS rings of 3 stages for K and for V^T.  K of tile i is read by the steps
// of halves (i-1, 1) and (i, 0) (scores one half ahead), V^T of tile i by the
// steps of halves (i, 1) and (i+1, 0) (output products one half behind); the
// barrier after half (i, 0) frees the stages of K(i) and V^T(i-1), which then
// take K(i+3) and V^T(i+2): every tile load has two tiles of work to land in.
// The tile loop is unrolled by three, so every stage offset is a constant.
constexpr int kStages = 3;
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

// A walk over the key tiles of one split, one tile at a time (all scalar):
// patch tiles page by page through the visible table (the page id read once
// per page), then the special stream's tiles.  The number of patch tiles npt
// and tiles per whole page tpp are the split's (passed in, not stored).  When
// some visible page holds fewer tokens than a whole grid, tpre (the running
// key-tile counts of the visible pages, else null) gives each page its own
// ceil(len / 64) tiles, so no tile past a page's tokens is walked.
// (readfirstlane keeps every field in scalar registers: the integer
// division would otherwise come back in a vector register, and the page id
// with it, turning each tile load into a loop over lanes.)
struct TileWalk {
    int t, pi, tip, page, ntp;   // ntp: tiles of page pi
    __device__ void init(int t0, int npt, int tpp, cint_ptr vis, cint_ptr tpre) {
        t = uniform(t0);
        pi = uniform(t / tpp);   // a page holds at most tpp tiles: at or before t's page
        if (tpre && t < npt)
            while (t >= uniform(tpre[pi + 1])) pi = uniform(pi + 1);
        tip = uniform(tpre ? t - (t < npt ? uniform(tpre[pi]) : 0) : t - pi * tpp);
        ntp = tpre && t < npt ? uniform(tpre[pi + 1] - tpre[pi]) : tpp;
        page = t < npt ? uniform(vis[pi]) : 0;
    }
    // returns true when the walk enters a new patch page
    __device__ bool next(int npt, int tpp, cint_ptr vis, cint_ptr tpre) {
        ++t;
        if (++tip == ntp) {
            tip = 0;
            ++pi;
            if (t < npt) {
                page = uniform(vis[pi]);
                if (tpre) ntp = uniform(tpre[pi + 1] - tpre[pi]);
                return true;
            }
        }
        return false;
    }
};

// Two 16-byte-per-lane tile loads straight into LDS (rows 8 apart: LDS
// addresses lds0 and lds0 + 1024), written as one asm statement so that the
// compiler does not track them: it would otherwise wait for them before
// operand reads of other stages it cannot tell apart.  The tile loop orders
// them itself (s_waitcnt vmcnt(0) and a barrier before any read of the stage
// they fill).  M0 carries the LDS address of an LDS DMA; it is saved and
// restored around the loads, with the wait states a write of M0 needs before
// such a load.  The loads write no VGPR.
__device__ inline void dma_pair(__amdgpu_buffer_rsrc_t r, const char* lds0, uint32_t voff0, uint32_t voff1,
                                uint32_t soff) {
    const uint32_t a0 = (uint32_t)uniform((int)(uint32_t)(uintptr_t)lds0);
    const uint32_t a1 = a0 + 1024u;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 1\n\t"
        "buffer_load_dwordx4 %3, %5, %6 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 1\n\t"
        "buffer_load_dwordx4 %4, %5, %6 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(a0), "s"(a1), "v"(voff0), "v"(voff1), "s"(r), "s"(soff)
        : "memory");
}

// Loads of one (stream, head): buffer resources over its K pool, V^T pool and
// special K / V^T, and this lane's byte offsets inside the 8-row slabs it
// loads (its row, and the 16-byte chunk that belongs at its slot under the
// swizzle).  A wave loads rows 16*wave .. 16*wave+15 of a tile, 8 rows per
// load.
struct Loader {
    __amdgpu_buffer_rsrc_t kpool, vpool, ksp, vsp;
    cint_ptr vis;            // visible pages
    int slot_cap;
    uint32_t lk0, lk1, lvp0, lvp1, lvs0, lvs1;

    __device__ void issue_k(const TileWalk& w, int npt, char* stage, int wave) const {
        const char* d = stage + wave * 2 * 8 * 128;
        if (w.t < npt) {
            const uint32_t ko = ((uint32_t)w.page * (uint32_t)slot_cap + (uint32_t)w.tip * kTile) * 128u;
            dma_pair(kpool, d, lk0, lk1, ko);
        } else {
            dma_pair(ksp, d, lk0, lk1, (uint32_t)(w.t - npt) * kTile * 128u);
        }
    }
    __device__ void issue_v(const TileWalk& w, int npt, char* stage, int wave) const {
        const char* d = stage + wave * 2 * 8 * 128;
        if (w.t < npt) {
            const uint32_t vo = (uint32_t)w.page * (uint32_t)slot_cap * 128u + (uint32_t)w.tip * kTile * 2u;
            dma_pair(vpool, d, lvp0, lvp1, vo);
        } else {
            dma_pair(vsp, d, lvs0, lvs1, (uint32_t)(w.t - npt) * kTile * 2u);
        }
    }
};

// Running state of one wave's 32 queries.
struct Acc {
    f32x16 o0, o1;     // O^T, d rows 0-31 and 32-63
    f32x4 rs;          // row sums: lanes 0-15 hold those of queries lane (rs[0]) and lane+16 (rs[1])
    float M;           // reference max of the base-2 exponents (shared by lanes l and l^32)
    float c;           // log2(e)/sqrt(D)
};

// s = q.k + init for the 32 keys of half kb of a tile (rows 32*kb + col of
// the K tile; chunk 2*j + hh is k-step j).  init is the accumulator's start:
// 0 for a key that counts, -inf for one past the end of a ragged half, so the
// mask costs nothing in the steps.
__device__ __forceinline__ f32x16 scores(const char* tile, int kb, const int* foff, const bf16x8* qf,
                                         const f32x16& init) {
    const char* t = tile + kb * kHalfBytes;
    const bf16x8 k0 = *(const bf16x8*)(t + foff[0]);
    const bf16x8 k1 = *(const bf16x8*)(t + foff[1]);
    const bf16x8 k2 = *(const bf16x8*)(t + foff[2]);
    const bf16x8 k3 = *(const bf16x8*)(t + foff[3]);
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[0], init, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[1], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k2, qf[2], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k3, qf[3], s, 0, 0, 0);
    return s;
}

// Output products and row sums of a half whose bf16 weights are pp (V^T rows
// of half vkb of the tile at vt).
__device__ __forceinline__ void products(const bf16x8 (&pp)[2], const char* vt, int vkb, const int* foff,
                                         const bf16x8& sel, Acc& A) {
    bf16x8 v[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        v[m][0] = *(const bf16x8*)(vt + foff[2 * vkb + m]);
        v[m][1] = *(const bf16x8*)(vt + kHalfBytes + foff[2 * vkb + m]);
    }
    A.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[0][0], pp[0], A.o0, 0, 0, 0);
    A.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[0][1], pp[0], A.o1, 0, 0, 0);
    A.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[1][0], pp[1], A.o0, 0, 0, 0);
    A.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[1][1], pp[1], A.o1, 0, 0, 0);
    A.rs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pp[0], A.rs, 0, 0, 0);
    A.rs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pp[1], A.rs, 0, 0, 0);
}

// p = exp2(s*c - M) of the 16 scores, rounded to bf16 and packed as the two
// 16-key operand blocks of the half (keys 0-15 from sc[0..7], 16-31 from
// sc[8..15]).
__device__ __forceinline__ void weights(const f32x16& sc, float c, float M, bf16x8 (&pn)[2]) {
    bf16x2 pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const f32x2 x = {__builtin_amdgcn_exp2f(fmaf(sc[2 * e], c, -M)),
                         __builtin_amdgcn_exp2f(fmaf(sc[2 * e + 1], c, -M))};
        pr[e] = __builtin_convertvector(x, bf16x2);
    }
    pn[0] = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                    __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    pn[1] = __builtin_shufflevector(__builtin_shufflevector(pr[4], pr[5], 0, 1, 2, 3),
                                    __builtin_shufflevector(pr[6], pr[7], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// One pipeline step: the softmax weights pn of the half whose scores are sc
// (keys past a ragged half's end already at -inf), the scores sn of the next
// half (K rows at knext, accumulator started at init) and the output products
// of the previous half (weights pp, V^T half vkb of the tile at vprev).  Key of
// sc[r]: 8*(r/4) + 4*hh + r%4 within the half.  No branch but the rare
// rescale, so the operand reads of the step overlap its products.
__device__ __forceinline__ void step(f32x16& sc, f32x16& sn, bf16x8 (&pn)[2], const bf16x8 (&pp)[2],
                                     const char* knext, const char* vprev, int vkb, const f32x16& init,
                                     const int* foff, const bf16x8* qf, const bf16x8& sel, Acc& A) {
    sn = scores(knext, 0, foff, qf, init);
    products(pp, vprev, vkb, foff, sel, A);
    weights(sc, A.c, A.M, pn);
    // M is kept 7 above the largest exponent seen when it last moved, so the
    // weights stay below 2^-7 until a score exceeds that max by 8 (base 2).
    // Some weight >= 2 (bf16 exponent field >= 128: its top bit set), or the
    // first valid keys against the initial M: move M to 7 above this half's
    // max (jointly for the two lanes of a query; never down), rescale what
    // was accumulated -- including the products just issued, which used the
    // old M -- and form the weights again.
    const u32x4 w0 = __builtin_bit_cast(u32x4, pn[0]);
    const u32x4 w1 = __builtin_bit_cast(u32x4, pn[1]);
    const uint32_t any = (w0[0] | w0[1] | w0[2]) | (w0[3] | w1[0] | w1[1]) | (w1[2] | w1[3]);
    if (__builtin_expect(__any((any & 0x40004000u) != 0u), 0)) {
        const float ma = max3f(sc[0], sc[1], sc[2]);
        const float mb = max3f(sc[3], sc[4], sc[5]);
        const float mc = max3f(sc[6], sc[7], sc[8]);
        const float md = max3f(sc[9], sc[10], sc[11]);
        const float me = max3f(sc[12], sc[13], sc[14]);
        const float mx = max3f(max3f(ma, mb, mc), fmaxf(md, me), sc[15]);
        const float m_new = fmaxf(fmaf(fmaxf(mx, __shfl_xor(mx, 32)), A.c, 7.f), A.M);
        const float alpha = __builtin_amdgcn_exp2f(A.M - m_new);
        A.M = m_new;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            A.o0[r] *= alpha;
            A.o1[r] *= alpha;
        }
        // rs[0] of lane n is query n's (alpha of this lane), rs[1] query n+16's
        A.rs[0] *= alpha;
        A.rs[1] *= __shfl_down(alpha, 16);
        weights(sc, A.c, A.M, pn);
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attend_bf16(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char ring[2 * kStages * kTileBytes];
    __shared__ int s_vlen[kMaxPool];   // tokens of each visible patch page
    char* const k0 = ring;
    char* const k1 = ring + kTileBytes;
    char* const k2 = ring + 2 * kTileBytes;
    char* const v0 = ring + 3 * kTileBytes;
    char* const v1 = ring + 4 * kTileBytes;
    char* const v2 = ring + 5 * kTileBytes;

    // Logical workgroup id: consecutive physical ids go round-robin to the 8
    // XCDs, so the remap gives each XCD a contiguous range of logical ids; the
    // q-tiles of one (stream, head, split) share their K/V tiles in that XCD's L2.
    const int per_xcd = gridDim.x / 8;
    const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (L >= a.n_logical) return;
    // (all uniform: kept in scalar registers, so the cache state and the
    // visible table are read through the scalar cache)
    const int qt = uniform(L % a.q_tiles);
    int rest = uniform(L / a.q_tiles);
    const int split = uniform(rest % a.splits);
    rest = uniform(rest / a.splits);
    const int h = uniform(rest % a.H);
    const int s = uniform(rest / a.H);

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
    ld.vis = (cint_ptr)(uintptr_t)st->vis;
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
    // Pages that hold fewer tokens than a whole grid: walk their own tiles
    // only (running counts written with the visible table).
    const bool vis_full = uniform(st->vis_full) != 0;
    const cint_ptr tpre = vis_full ? nullptr : (cint_ptr)(uintptr_t)st->vis_tpre;
    const int n_patch_tiles = vis_full ? vis_n * a.tpp : uniform(tpre[vis_n]);
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
    // Selection operand of the row sums (A of v_mfma_f32_16x16x32_bf16, lane
    // l holds row l%16, k-columns 8*(l/16)..+7): a P^T block used as the B
    // operand puts the keys of query n in k-groups 0 and 2 and those of query
    // n+16 in groups 1 and 3 (column n), so row 0 sums query n, row 1 query n+16.
    bf16x8 sel;
    {
        const int m = lane & 15, g = lane >> 4;
        const __bf16 v = (__bf16)(((m == 0 && (g & 1) == 0) || (m == 1 && (g & 1) == 1)) ? 1.f : 0.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) sel[i] = v;
    }

    Acc A;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        A.o0[i] = 0.f;
        A.o1[i] = 0.f;
    }
    A.rs = f32x4{0.f, 0.f, 0.f, 0.f};
    // A finite start far below any score: the first valid weights come out
    // infinite, which moves M to their max.
    A.M = -1e30f;
    A.c = a.scale_log2;

    // Operand byte offsets inside a tile ((row >> 1) & 7 == (col >> 1) & 7 for
    // every 32-row block).
    int foff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) foff[j] = col * 128 + (((2 * j + hh) ^ ((col >> 1) & 7)) << 4);

    // Page lengths: all P when every visible page holds a whole grid (then
    // nothing is read per tile), else an LDS copy.
    if (!vis_full)
        for (int i = tid; i < vis_n; i += 256) s_vlen[i] = st->vis_len[i];
    auto page_len = [&](int pi) { return vis_full ? a.P : uniform(s_vlen[pi]); };

    __syncthreads();   // publishes s_vlen

    if (n > 0) {
        // Two walks: wk issues K tiles three ahead, wv issues V^T tiles two
        // ahead and gives the valid keys of the tile it is at (a patch page
        // holds the tokens its frame had, the special stream vis_sp).
        const int npt = n_patch_tiles, tpp = a.tpp;
        TileWalk wk, wv;
        wk.init(t0, npt, tpp, ld.vis, tpre);
        wv = wk;
        int plen = wv.t < npt ? page_len(wv.pi) : 0;   // tokens of wv's page
        auto tile_len = [&]() {
            return wv.t < npt ? min(kTile, plen - wv.tip * kTile) : min(kTile, vis_sp - (wv.t - npt) * kTile);
        };
        auto next_v = [&]() {
            if (wv.next(npt, tpp, ld.vis, tpre)) plen = page_len(wv.pi);
        };
        // Prologue: K(0..2) and V^T(0..1); the V^T stage the first step's
        // (empty) products read is zeroed so that stale LDS contents cannot
        // reach them.
        ld.issue_k(wk, npt, k0, wave);
        wk.next(npt, tpp, ld.vis, tpre);
        if (n > 1) {
            ld.issue_k(wk, npt, k1, wave);
            wk.next(npt, tpp, ld.vis, tpre);
        }
        if (n > 2) {
            ld.issue_k(wk, npt, k2, wave);
            wk.next(npt, tpp, ld.vis, tpre);
        }
        int la = 0, lb = 0, lc = 0;   // valid keys of tiles i, i+1, i+2 (rotating)
        ld.issue_v(wv, npt, v0, wave);
        la = tile_len();
        next_v();
        if (n > 1) {
            ld.issue_v(wv, npt, v1, wave);
            lb = tile_len();
            next_v();
        }
        *(uint4*)(v2 + tid * 16) = make_uint4(0, 0, 0, 0);
        *(uint4*)(v2 + 4096 + tid * 16) = make_uint4(0, 0, 0, 0);
        wait_vmcnt<0>();
        __syncthreads();

        // Accumulator start of the next score products: zero, or -inf on the
        // keys past the end of a ragged half (set only when one comes).
        f32x16 init = {};
        bool masked = false;
        auto set_init = [&](int len, int kb) {   // for half kb of a tile of len valid keys
            const int lim = len - 32 * kb - 4 * hh;
            if (len >= 32 * kb + 32) {
                if (masked) {
                    init = f32x16{};
                    masked = false;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) init[r] = 8 * (r >> 2) + (r & 3) >= lim ? -INFINITY : 0.f;
                masked = true;
            }
        };
        set_init(la, 0);
        f32x16 sa = scores(k0, 0, foff, qf, init), sb;
        bf16x8 pa[2], pb[2];
        pb[0] = bf16x8{};
        pb[1] = bf16x8{};
        // half (0, 0): scores of (0, 1), (empty) products against the zeroed stage
        set_init(la, 1);
        step(sa, sb, pa, pb, k0 + kHalfBytes, v2, 1, init, foff, qf, sel, A);
        __syncthreads();
        // From the barrier after half (i, 0), with K(i) in kc, K(i+1) in kn,
        // V^T(i) in vc and V^T(i-1) in vp, and the valid keys of tiles i,
        // i+1, i+2 in lcur, lnext, lnext2: the stages of K(i) and V^T(i-1)
        // take K(i+3) and V^T(i+2); half (i, 1); half (i+1, 0); then the
        // barrier after it, once the loads issued at the previous barrier
        // (K(i+2), V^T(i+1)) have landed.  Returns false after the last tile.
        auto tile = [&](int i, char* kc, char* kn, char* vc, char* vp, int& lcur, int& lnext,
                        int& lnext2) {
            int issued = 0;   // loads of this wave in flight from this barrier
            if (i + 3 < n) {
                ld.issue_k(wk, npt, kc, wave);
                wk.next(npt, tpp, ld.vis, tpre);
                issued += 2;
            }
            if (i + 2 < n) {
                ld.issue_v(wv, npt, vp, wave);
                lnext2 = tile_len();
                next_v();
                issued += 2;
            }
            // half (i, 1): scores of (i+1, 0) (past the last tile: a stale
            // stage, never used), products of (i, 0)
            set_init(lnext, 0);
            step(sb, sa, pb, pa, kn, vc, 0, init, foff, qf, sel, A);
            if (i + 1 == n) return false;
            // half (i+1, 0): scores of (i+1, 1), products of (i, 1)
            set_init(lnext, 1);
            step(sa, sb, pa, pb, kn + kHalfBytes, vc, 1, init, foff, qf, sel, A);
            if (issued == 4)
                wait_vmcnt<4>();
            else if (issued == 2)
                wait_vmcnt<2>();
            else
                wait_vmcnt<0>();
            __syncthreads();
            return true;
        };
        for (int i = 0;; i += 3) {
            if (!tile(i, k0, k1, v0, v2, la, lb, lc)) break;
            if (!tile(i + 1, k1, k2, v1, v0, lb, lc, la)) break;
            if (!tile(i + 2, k2, k0, v2, v1, lc, la, lb)) break;
        }
        // products of the last half
        const int last = (n - 1) % 3;
        products(pb, last == 0 ? v0 : last == 1 ? v1 : v2, 1, foff, sel, A);
    }

    // Row sum of the lane's query (rows 0 / 1 of the row-sum block, lanes
    // 0-15); output O = O^T / l.
    const float l0 = __shfl(A.rs[0], col & 15);
    const float l1 = __shfl(A.rs[1], col & 15);
    const float l = col < 16 ? l0 : l1;
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
