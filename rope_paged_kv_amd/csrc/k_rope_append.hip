// Fused 3D rotary embedding + paged KV append + bookkeeping commit.
//
// What is computed (page "How 3D RoPE Positional Encoding Works with the
// Paged KV Cache in LingBot-Map": "Complex-Valued Tensor Application",
// "Frame Appending and Position Encoding Integration", "Dual-Stream Memory
// Layout", "Attention Computation with Cached RoPE"; page "KV Caching Benefits
// in Ling Bot-Map": "Reduced KV Growth via Keyframe Streaming"):
//  * every (x[2j], x[2j+1]) pair of Q and K is rotated by the angle of its
//    token's (t, h, w) position on the pair's axis -- a complex product done
//    in real fp32 arithmetic, rounded once to the storage dtype;
//  * rotated K and raw V of the patch tokens go to the frame's patch page,
//    those of the special tokens to the special stream; rotated Q goes to
//    q_rot for the attention kernel;
//  * the target page is the free-list top, else the next never-used page, and
//    the specials go right after the committed ones: the frame's tentative
//    slot; the deferred-eviction call later keeps it (keyframe) or not
//    (skip-append);
//  * the visible page table is rebuilt: scale pages, window pages oldest
//    first, the frame's own page, then the special pages and the last special
//    page's length.
//
// Layout of the work: one workgroup per (tile of 64 tokens, head, stream);
// tile 0 carries the special tokens.  Each thread moves 16-byte chunks, so
// every row (one token of one head, 128 B in bf16) is read and written with
// full-width coalesced accesses; V goes through LDS to be written transposed
// (the layout the attention kernel's matrix-core operands read).  The
// bookkeeping never leaves the device: every workgroup derives the target page
// from the state as it stands (which no workgroup of the launch modifies), and
// one workgroup per stream writes the frame record -- no atomics, no fences.
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

// Rotation coefficients (cos, sin) of pair j of a token at grid position
// (hp, wp): the t table for j < pt, the h table for the next ph pairs and the
// w table after that.
__device__ inline float2 coeff(const AppendArgs& a, int j, int hp, int wp) {
    const float2* src = j < a.pt ? a.tab_t + a.frame * a.pt + j
                      : j < a.pt + a.ph ? a.tab_h + hp * a.ph + (j - a.pt)
                                        : a.tab_w + wp * a.pw + (j - a.pt - a.ph);
    return *src;
}

// Row and 16-byte chunk of a thread's chunk slot i.  Interleaved layout:
// slots walk the tile's chunks in order.  Half-split layout: slots 2j and
// 2j+1 are a pair of chunks that rotate together -- a chunk of the first half
// of an axis block and the chunk pairs_a channels after it -- and the pair
// slots walk the tile's first-half chunks in order (cpr/2 per row).
template <int CH, int LAYOUT>
__device__ inline void chunk_of(const AppendArgs& a, int tid, int i, int& r, int& c) {
    constexpr int CPR = kHeadDim / CH;
    if (LAYOUT == RPKV_ROPE_INTERLEAVED) {
        const int id = tid + i * 256;
        r = id / CPR;
        c = id % CPR;
        return;
    }
    const int id = tid + (i >> 1) * 256;
    r = id / (CPR / 2);
    int pc = id % (CPR / 2);
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
    c = base + pc + ((i & 1) ? half : 0);
}

// Rotation coefficients of a thread's chunk slots, flat: interleaved, pair e
// of slot i at [i*CH/2 + e]; half-split, channel e of pair slot j at [j*CH + e].
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

template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void k_rope_append(AppendArgs a) {
    constexpr int CH = Vec<T>::kCh;        // elements per 16-byte chunk
    constexpr int CPR = kHeadDim / CH;     // chunks per row
    constexpr int NCH = kTile * CPR;       // chunks per tile and tensor
    constexpr int PER = NCH / 256;         // chunks per thread
    __shared__ T vt[kHeadDim][kTile + CH]; // V^T of the tile: row d, storage position

    const int tile = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
    CacheState* st = a.states + s;

    const bool special = tile == 0;
    const int slot0 = special ? 0 : (tile - 1) * kTile;
    const int nrows = special ? a.nsp : min(kTile, a.fP - slot0);   // may be <= 0: a tile past the frame's patches
    const int tok0 = special ? 0 : a.nsp + slot0;

    const size_t rs = (size_t)a.H * kHeadDim;  // elements between consecutive tokens
    const size_t in_off = ((size_t)s * a.N + tok0) * rs + (size_t)h * kHeadDim;
    const T* qb = (const T*)a.q + in_off;
    const T* kb = (const T*)a.k + in_off;
    const T* vb = (const T*)a.v + in_off;
    T* qrb = (T*)a.q_rot + in_off;

    // Every load first, none waiting on another: this thread's chunks of Q,
    // K and V (rows past the tile's tokens read row 0 and are dropped), then
    // the rotation coefficients of its pairs.  The bookkeeping state, read
    // next through the scalar cache, only decides where the results go.
    uint4 qv[PER], kv[PER], vv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int r, c;
        chunk_of<CH, LAYOUT>(a, tid, i, r, c);
        const size_t off = (size_t)(r < nrows ? r : 0) * rs + c * CH;
        qv[i] = *(const uint4*)(qb + off);
        kv[i] = *(const uint4*)(kb + off);
        vv[i] = *(const uint4*)(vb + off);
    }
    float2 cs[PER * CH / 2];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int r, c;
        chunk_of<CH, LAYOUT>(a, tid, i, r, c);
        int hp = 0, wp = 0;   // specials sit at h = w = 0
        if (!special) {
            const int p = r < nrows ? slot0 + r : 0;   // rows past the frame's patches: (0, 0)
            hp = p / a.fgw;
            wp = p - hp * a.fgw;
        }
        if (LAYOUT == RPKV_ROPE_INTERLEAVED) {
#pragma unroll
            for (int e = 0; e < CH / 2; ++e) cs[i * (CH / 2) + e] = coeff_of<CH, LAYOUT>(a, c, e, hp, wp);
        } else if ((i & 1) == 0) {
#pragma unroll
            for (int e = 0; e < CH; ++e) cs[(i >> 1) * CH + e] = coeff_of<CH, LAYOUT>(a, c, e, hp, wp);
        }
    }

    // Target of this append, from the state as it stands.
    const int status = st->status;
    const int n_free = st->n_free;
    const int fresh = st->fresh;
    const int page = n_free > 0 ? st->free_[n_free - 1] : fresh;
    const int sp_off = st->n_sp;
    // The special stream always has room for one frame beyond the committed
    // ones; its capacity is checked when the frame is committed.
    const bool ok = status == RPKV_OK && (n_free > 0 || fresh < a.pool);
    T* kdst;
    if (special)
        kdst = (T*)a.ksp + s * a.ksp_elems + ((size_t)h * a.sp_cap + sp_off) * kHeadDim;
    else
        kdst = (T*)a.kpool + s * a.kpool_elems +
               (((size_t)h * a.pool + page) * a.slot_cap + slot0) * kHeadDim;

    // Rotate (a complex product per pair in fp32, rounded once), store Q and
    // K; V goes to LDS transposed, at its storage position.
    float fq[PER][CH], fk[PER][CH];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        Vec<T>::unpack(qv[i], fq[i]);
        Vec<T>::unpack(kv[i], fk[i]);
    }
    if (LAYOUT == RPKV_ROPE_INTERLEAVED) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int e = 0; e < CH / 2; ++e) {
                const float2 w = cs[i * (CH / 2) + e];
                const float xq = fq[i][2 * e], yq = fq[i][2 * e + 1];
                fq[i][2 * e] = xq * w.x - yq * w.y;
                fq[i][2 * e + 1] = xq * w.y + yq * w.x;
                const float xk = fk[i][2 * e], yk = fk[i][2 * e + 1];
                fk[i][2 * e] = xk * w.x - yk * w.y;
                fk[i][2 * e + 1] = xk * w.y + yk * w.x;
            }
    } else {
#pragma unroll
        for (int j = 0; j < PER / 2; ++j)
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float2 w = cs[j * CH + e];
                const float xq = fq[2 * j][e], yq = fq[2 * j + 1][e];
                fq[2 * j][e] = xq * w.x - yq * w.y;
                fq[2 * j + 1][e] = yq * w.x + xq * w.y;
                const float xk = fk[2 * j][e], yk = fk[2 * j + 1][e];
                fk[2 * j][e] = xk * w.x - yk * w.y;
                fk[2 * j + 1][e] = yk * w.x + xk * w.y;
            }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int r, c;
        chunk_of<CH, LAYOUT>(a, tid, i, r, c);
        const bool valid = r < nrows;
        if (valid) {
            *(uint4*)(qrb + r * rs + c * CH) = Vec<T>::pack(fq[i]);
            if (ok) *(uint4*)(kdst + r * kHeadDim + c * CH) = Vec<T>::pack(fk[i]);
        }
        // Rows past the tile's tokens are zeros (padding slots stay zero).
        const uint4 v = valid ? vv[i] : make_uint4(0, 0, 0, 0);
        const T* ve = (const T*)&v;
        const int pos = special ? r : vslot_perm(r);
#pragma unroll
        for (int e = 0; e < CH; ++e) vt[c * CH + e][pos] = ve[e];
    }
    __syncthreads();

    if (ok) {
        if (!special) {
            // V^T rows d of the page, storage positions slot0 .. slot0+63.
            T* vdst = (T*)a.vpool + s * a.kpool_elems +
                      ((size_t)h * a.pool + page) * kHeadDim * a.slot_cap + slot0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int id = tid + i * 256;
                const int d = id / CPR, g = id % CPR;
                *(uint4*)(vdst + (size_t)d * a.slot_cap + g * CH) = *(const uint4*)&vt[d][g * CH];
            }
        } else {
            T* vdst = (T*)a.vsp + s * a.ksp_elems + (size_t)h * kHeadDim * a.sp_cap;
            for (int id = tid; id < a.nsp * kHeadDim; id += 256) {
                const int r = id / kHeadDim, d = id % kHeadDim;
                vdst[(size_t)d * a.sp_cap + vslot_perm(sp_off + r)] = vt[d][r];
            }
        }
    }

    // Frame record, written by one workgroup per stream: the visible table
    // this frame's attention reads, and the pending commit that the deferred
    // eviction call applies.  It touches only fields no workgroup of this
    // launch reads (the structural state above is left as it is), so no
    // workgroup waits for another.
    if (tile != 0 || h != 0) return;
    // Visible patch pages: scale pages, window oldest first, then the frame's
    // own page (it comes last whether it will be committed or not).
    const int ns = st->n_scale, nw = st->n_win, head = st->win_head;
    const int vis_n = ok ? ns + nw + 1 : 0;
    int full = 1;
    for (int i = tid; i < vis_n; i += 256) {
        const int pg = i < ns ? st->scale[i] : (i < ns + nw ? st->win[(head + i - ns) % kMaxPool] : page);
        st->vis[i] = pg;
        const int len = i < ns + nw ? st->page_tokens[pg] : a.fP;
        st->vis_len[i] = len;
        full &= len == a.P;
    }
    full = __syncthreads_and(full);
    if (tid == 0) {
        st->n_query = a.nsp + a.fP;
        st->vis_full = full;
        if (!ok) {
            if (status == RPKV_OK) st->status = RPKV_ENOSPACE;
            st->vis_n = 0;
            st->vis_sp_tokens = 0;
            st->vis_sp_pages = 0;
            st->last_page_len = 0;
            st->pending = 0;
        } else {
            const int vis_sp = sp_off + a.nsp;
            const int sp_pages = (vis_sp + a.sp_page - 1) / a.sp_page;
            st->target = page;
            st->sp_off = sp_off;
            st->page_tokens[page] = a.fP;
            st->vis_n = vis_n;
            st->vis_sp_tokens = vis_sp;
            st->vis_sp_pages = sp_pages;
            st->last_page_len = sp_pages ? vis_sp - (sp_pages - 1) * a.sp_page : 0;
            st->pending = a.commit;
        }
    }
}

hipError_t launch_rope_append(const AppendArgs& a, int dtype, hipStream_t st) {
    dim3 grid(a.n_tiles, a.H, a.S);
    const bool half = a.layout == RPKV_ROPE_HALF_SPLIT;
    if (dtype == RPKV_BF16) {
        if (half)
            hipLaunchKernelGGL((k_rope_append<uint16_t, RPKV_ROPE_HALF_SPLIT>), grid, dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL((k_rope_append<uint16_t, RPKV_ROPE_INTERLEAVED>), grid, dim3(256), 0, st, a);
    } else {
        if (half)
            hipLaunchKernelGGL((k_rope_append<float, RPKV_ROPE_HALF_SPLIT>), grid, dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL((k_rope_append<float, RPKV_ROPE_INTERLEAVED>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace rpkv
