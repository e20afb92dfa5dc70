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
// full-width coalesced accesses (in the half-split layout a chunk's rotation
// partner is read from the lane that loaded it); V goes through LDS to be
// written transposed
// (the layout the attention kernel's matrix-core operands read).  The
// bookkeeping never leaves the device: every workgroup derives the target page
// from the state as it stands (which no workgroup of the launch modifies), and
// one extra workgroup per stream, the first of its row of the grid, writes the
// frame record -- no atomics, no fences.
#include "rope_rows.h"

namespace rpkv {

template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void k_rope_append(AppendArgs a) {
    constexpr int CH = Vec<T>::kCh;        // elements per 16-byte chunk
    constexpr int CPR = kHeadDim / CH;     // chunks per row
    constexpr int NCH = kTile * CPR;       // chunks per tile and tensor
    constexpr int PER = NCH / 256;         // chunks per thread
    __shared__ T vt[kHeadDim][kTile + CH]; // V^T of the tile: row d, storage position

    const int h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
    CacheState* st = a.states + s;
    // Workgroup x = 0 of head 0 writes the frame record and nothing else, so
    // its chain of dependent bookkeeping loads starts with the launch instead
    // of trailing a tile's work; x = 0 of the other heads has nothing to do.
    if (blockIdx.x == 0) {
        if (h == 0) write_frame_record(a, st, append_target(a, st), tid);
        return;
    }
    const int tile = blockIdx.x - 1;

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
        chunk_of<CH>(tid, i, r, c);
        const size_t off = (size_t)(r < nrows ? r : 0) * rs + c * CH;
        qv[i] = *(const uint4*)(qb + off);
        kv[i] = *(const uint4*)(kb + off);
        vv[i] = *(const uint4*)(vb + off);
    }
    // interleaved: pair e of slot i at [i*CH/2 + e]; half-split: the pair
    // of channel e of slot i at [i*CH + e]
    float2 cs[LAYOUT == RPKV_ROPE_INTERLEAVED ? PER * CH / 2 : PER * CH];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int r, c;
        chunk_of<CH>(tid, i, r, c);
        int hp = 0, wp = 0;   // specials sit at h = w = 0
        if (!special) {
            const int p = r < nrows ? slot0 + r : 0;   // rows past the frame's patches: (0, 0)
            hp = p / a.fgw;
            wp = p - hp * a.fgw;
        }
        if (LAYOUT == RPKV_ROPE_INTERLEAVED) {
#pragma unroll
            for (int e = 0; e < CH / 2; ++e) cs[i * (CH / 2) + e] = coeff_of<CH, LAYOUT>(a, c, e, hp, wp);
        } else {
            bool first;
            int dc, cf;
            half_partner<CH>(a, c, first, dc, cf);
#pragma unroll
            for (int e = 0; e < CH; ++e) cs[i * CH + e] = coeff_of<CH, LAYOUT>(a, cf, e, hp, wp);
        }
    }

    const Target tg = append_target(a, st);
    const int page = tg.page, sp_off = tg.sp_off;
    const bool ok = tg.ok;
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
        // The pair partner of a lane's chunk sits in the same row, so in the
        // same wave, dc lanes away: read across lanes, then each lane rotates
        // its own chunk (first half: x cos - y sin; second half: x cos + y sin,
        // x its own value and y the partner's).
        const int lane = tid & 63;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int r, c;
            chunk_of<CH>(tid, i, r, c);
            bool first;
            int dc, cf;
            half_partner<CH>(a, c, first, dc, cf);
            const int pl = lane + dc;
            const uint4 pq = make_uint4(__shfl((int)qv[i].x, pl), __shfl((int)qv[i].y, pl),
                                        __shfl((int)qv[i].z, pl), __shfl((int)qv[i].w, pl));
            const uint4 pk = make_uint4(__shfl((int)kv[i].x, pl), __shfl((int)kv[i].y, pl),
                                        __shfl((int)kv[i].z, pl), __shfl((int)kv[i].w, pl));
            float gq[CH], gk[CH];
            Vec<T>::unpack(pq, gq);
            Vec<T>::unpack(pk, gk);
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float2 w = cs[i * CH + e];
                const float xq = fq[i][e], yq = gq[e], xk = fk[i][e], yk = gk[e];
                fq[i][e] = first ? xq * w.x - yq * w.y : xq * w.x + yq * w.y;
                fk[i][e] = first ? xk * w.x - yk * w.y : xk * w.x + yk * w.y;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int r, c;
        chunk_of<CH>(tid, i, r, c);
        const bool valid = r < nrows;
        if (valid) {
            *(uint4*)(qrb + r * rs + c * CH) = Vec<T>::pack(fq[i]);
            if (ok) store_stream(kdst + r * kHeadDim + c * CH, Vec<T>::pack(fk[i]));
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
                store_stream(vdst + (size_t)d * a.slot_cap + g * CH, *(const uint4*)&vt[d][g * CH]);
            }
        } else {
            T* vdst = (T*)a.vsp + s * a.ksp_elems + (size_t)h * kHeadDim * a.sp_cap;
            for (int id = tid; id < a.nsp * kHeadDim; id += 256) {
                const int r = id / kHeadDim, d = id % kHeadDim;
                vdst[(size_t)d * a.sp_cap + vslot_perm(sp_off + r)] = vt[d][r];
            }
        }
    }
}

hipError_t launch_rope_append(const AppendArgs& a, int dtype, hipStream_t st) {
    dim3 grid(a.n_tiles + 1, a.H, a.S);   // x = 0: the frame record
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
