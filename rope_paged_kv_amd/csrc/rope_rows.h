// Pieces shared by the kernels that rotate a frame's Q and K and append it to
// the paged cache (k_rope_append, k_project_append): 16-byte chunk packing,
// the rotation coefficients of a chunk, the chunk pairing of the two channel
// layouts, the target of an append and the frame record.
//
// Rotation: page "How 3D RoPE Positional Encoding Works with the Paged KV
// Cache in LingBot-Map", "Complex-Valued Tensor Application"; half-split
// pairing: page "How to Handle Sequences Exceeding the RoPE Training Range in
// LingBot-Map", "Understanding the 2D RoPE Architecture".  Visible table:
// same first page, "Attention Computation with Cached RoPE".
#pragma once
#include "rpkv_internal.h"

namespace rpkv {

template <typename T>
struct Vec;

template <>
struct Vec<uint16_t> {   // bf16 bit patterns
    static constexpr int kCh = 8;
    __device__ static inline void unpack(const uint4& r, float* f) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static inline uint32_t pack2(float lo, float hi) {
        // round to nearest even (inputs are finite)
        uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
        a += 0x7FFFu + ((a >> 16) & 1u);
        b += 0x7FFFu + ((b >> 16) & 1u);
        return (a >> 16) | (b & 0xFFFF0000u);
    }
    __device__ static inline uint4 pack(const float* f) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
    }
};

template <>
struct Vec<float> {
    static constexpr int kCh = 4;
    __device__ static inline void unpack(const uint4& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    __device__ static inline uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

// 16-byte store that streams past the caches: the pages are read only by
// later frames' attention, not by anything in this launch or the next one.
__device__ inline void store_stream(void* dst, const uint4& v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4*)dst);
}

// Rotation coefficients (cos, sin) of pair j of a token at grid position
// (hp, wp): the t table for j < pt, the h table for the next ph pairs and the
// w table after that.
__device__ inline float2 coeff(const AppendArgs& a, int j, int hp, int wp) {
    const float2* src = j < a.pt ? a.tab_t + a.frame * a.pt + j
                      : j < a.pt + a.ph ? a.tab_h + hp * a.ph + (j - a.pt)
                                        : a.tab_w + wp * a.pw + (j - a.pt - a.ph);
    return *src;
}

// Half-split layout: chunk of the pc-th first-half chunk of a row (second = 0)
// or of the chunk pairs_a channels after it (second = 1).  The first-half
// chunks of a row are walked axis by axis (t, h, w).
template <int CH>
__device__ inline int pair_chunk(const AppendArgs& a, int pc, int second) {
    const int nt = a.pt / CH, nh = a.ph / CH, nw = a.pw / CH;   // first-half chunks per axis
    int base, half;
    if (pc < nt) {
        base = 0;
        half = nt;
    } else if ((pc -= nt) < nh) {
        base = 2 * nt;
        half = nh;
    } else {
        pc -= nh;
        base = 2 * (nt + nh);
        half = nw;
    }
    return base + pc + (second ? half : 0);
}

// Row and 16-byte chunk of a thread's chunk slot i (256 threads): the slots
// walk the tile's chunks in order, so the lanes of a wave cover whole rows
// and every access is a full-width coalesced row.
template <int CH>
__device__ inline void chunk_of(int tid, int i, int& r, int& c) {
    constexpr int CPR = kHeadDim / CH;
    const int id = tid + i * 256;
    r = id / CPR;
    c = id % CPR;
}

// Half-split layout: the rotation partner of chunk c of a row -- dc chunks
// away, the chunk pairs_a channels after c in its axis block (c in the first
// half) or before it -- and the first-half chunk of the pair, which names the
// pair's coefficients.
template <int CH>
__device__ inline void half_partner(const AppendArgs& a, int c, bool& first, int& dc, int& cfirst) {
    const int nt = a.pt / CH, nh = a.ph / CH, nw = a.pw / CH;   // first-half chunks per axis
    int base, half;
    if (c < 2 * nt) {
        base = 0;
        half = nt;
    } else if (c < 2 * (nt + nh)) {
        base = 2 * nt;
        half = nh;
    } else {
        base = 2 * (nt + nh);
        half = nw;
    }
    first = c - base < half;
    dc = first ? half : -half;
    cfirst = first ? c : c - half;
}

// Rotation coefficients of a thread's chunk slots, flat: interleaved, pair e
// of slot i; half-split, the pair of channel e of first-half chunk c.
template <int CH, int LAYOUT>
__device__ inline float2 coeff_of(const AppendArgs& a, int c, int e, int hp, int wp) {
    if (LAYOUT == RPKV_ROPE_INTERLEAVED) return coeff(a, c * (CH / 2) + e, hp, wp);
    // half-split: chunk c of the first half of its axis block; pair index
    // inside the axis = channel offset from the block start.
    const int nt = a.pt / CH, nh = a.ph / CH;
    if (c < 2 * nt) return a.tab_t[a.frame * a.pt + c * CH + e];
    if (c < 2 * (nt + nh)) return a.tab_h[hp * a.ph + (c - 2 * nt) * CH + e];
    return a.tab_w[wp * a.pw + (c - 2 * (nt + nh)) * CH + e];
}

// Where an append goes, from the state as it stands (no workgroup of an
// append launch changes it): the free-list top, else the next never-used
// page; the specials right after the committed ones.  The special stream
// always has room for one frame beyond the committed ones; its capacity is
// checked when the frame is committed.
struct Target {
    int status, page, sp_off;
    bool ok;
};

__device__ inline Target append_target(const AppendArgs& a, const CacheState* st) {
    Target t;
    t.status = st->status;
    const int n_free = st->n_free;
    const int fresh = st->fresh;
    t.page = n_free > 0 ? st->free_[n_free - 1] : fresh;
    t.sp_off = st->n_sp;
    t.ok = t.status == RPKV_OK && (n_free > 0 || fresh < a.pool);
    return t;
}

// The frame record, written by the 256 threads of one workgroup per stream:
// the visible table this frame's attention reads and the pending commit that
// the deferred-eviction call applies.  It touches only fields no workgroup of
// an append launch reads, so no workgroup waits for another.
__device__ inline void write_frame_record(const AppendArgs& a, CacheState* st, const Target& tg,
                                          int tid) {
    // Visible patch pages: scale pages, window oldest first, then the frame's
    // own page (it comes last whether it will be committed or not).
    const int ns = st->n_scale, nw = st->n_win, head = st->win_head;
    const int vis_n = tg.ok ? ns + nw + 1 : 0;
    // Thread tid takes pages 2 tid and 2 tid + 1 (at most kMaxPool = 512), then
    // the workgroup scans their key-tile counts (ceil(len / kTile)) into the
    // running counts the attention walks a split's tiles by.
    __shared__ int tiles_scan[256];
    int full = 1, own = 0, first_tiles = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = 2 * tid + k;
        if (i < vis_n) {
            const int pg = i < ns ? st->scale[i] : (i < ns + nw ? st->win[(head + i - ns) % kMaxPool] : tg.page);
            st->vis[i] = pg;
            const int len = i < ns + nw ? st->page_tokens[pg] : a.fP;
            st->vis_len[i] = len;
            full &= len == a.P;
            const int nt = (len + kTile - 1) / kTile;
            if (k == 0) first_tiles = nt;
            own += nt;
        }
    }
    tiles_scan[tid] = own;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {   // inclusive scan (Hillis-Steele)
        const int v = tid >= off ? tiles_scan[tid - off] : 0;
        __syncthreads();
        tiles_scan[tid] += v;
        __syncthreads();
    }
    const int before = tiles_scan[tid] - own;   // tiles of pages 0 .. 2 tid - 1
    if (2 * tid <= vis_n) st->vis_tpre[2 * tid] = before;
    if (2 * tid + 1 <= vis_n) st->vis_tpre[2 * tid + 1] = before + first_tiles;
    if (tid == 255) st->vis_tpre[vis_n] = tiles_scan[255];   // the total (also for vis_n = 512)
    full = __syncthreads_and(full);
    if (tid == 0) {
        st->n_query = a.nsp + a.fP;
        st->vis_full = full;
        if (!tg.ok) {
            if (tg.status == RPKV_OK) st->status = RPKV_ENOSPACE;
            st->vis_n = 0;
            st->vis_sp_tokens = 0;
            st->vis_sp_pages = 0;
            st->last_page_len = 0;
            st->pending = 0;
        } else {
            const int vis_sp = tg.sp_off + a.nsp;
            const int sp_pages = (vis_sp + a.sp_page - 1) / a.sp_page;
            st->target = tg.page;
            st->sp_off = tg.sp_off;
            st->page_tokens[tg.page] = a.fP;
            st->vis_n = vis_n;
            st->vis_sp_tokens = vis_sp;
            st->vis_sp_pages = sp_pages;
            st->last_page_len = sp_pages ? vis_sp - (sp_pages - 1) * a.sp_page : 0;
            st->pending = a.commit;
        }
    }
}

}  // namespace rpkv
