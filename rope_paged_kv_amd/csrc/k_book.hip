// Cache bookkeeping kernels: zero fill, reset, commit + deferred eviction,
// rollback.
//
// Deferred eviction follows "KV Caching Benefits in Ling Bot-Map", sections
// "Memory-Efficient Sliding Window Management" (eviction runs once the frame
// has been processed) and "Dynamic Keyframe Selection" (the deferred-eviction
// call is what retains a keyframe's KV; a rollback drops the temporary entry),
// and "How 3D RoPE Positional Encoding Works with the Paged KV Cache in
// LingBot-Map", section "Dual-Stream Memory Layout" (the oldest window page
// goes back to the free list; scale pages and the special stream are never
// evicted).
#include "rpkv_internal.h"

namespace rpkv {

// Zero fill with 16-byte stores (used instead of hipMemsetAsync so that the
// fill is an ordinary kernel node when a caller captures it in a graph).
__global__ void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
    if (i < ntail) tail[i] = 0;
}

__global__ void k_reset(CacheState* states, int count) {
    int c = blockIdx.x;
    if (c >= count) return;
    CacheState* s = states + c;
    for (int i = threadIdx.x; i < kMaxPool; i += blockDim.x) s->page_tokens[i] = 0;
    if (threadIdx.x != 0) return;
    s->n_query = 0;
    s->pending = 0;
    s->status = RPKV_OK;
    s->fresh = 0;
    s->n_free = 0;
    s->n_scale = 0;
    s->win_head = 0;
    s->n_win = 0;
    s->n_sp = 0;
    s->target = -1;
    s->sp_off = 0;
    s->vis_n = 0;
    s->vis_sp_pages = 0;
    s->last_page_len = 0;
    s->vis_sp_tokens = 0;
}

// Deferred eviction, one workgroup per cache: first the pending commit of the
// last appended frame (a keyframe's page joins the scale list while it has
// fewer than scale_frames pages, else the window; its special tokens join the
// special stream), then the oldest window pages go to the free list while the
// window holds more than sliding_window pages.  The target page is still the
// free-list top (or the next never-used page): nothing changed it since the
// append.
__global__ void k_evict(CacheState* states, int count, int scale_frames, int sliding_window,
                        int max_sp_tokens, int nsp) {
    int c = blockIdx.x;
    if (c >= count || threadIdx.x != 0) return;
    CacheState* s = states + c;
    if (s->status != RPKV_OK) return;
    int n_win = s->n_win, head = s->win_head, n_free = s->n_free;
    if (s->pending) {
        s->pending = 0;
        if (s->n_sp + nsp > max_sp_tokens) {
            s->status = RPKV_ENOSPACE;
            return;
        }
        const int page = s->target;
        if (n_free > 0)
            --n_free;
        else
            s->fresh = s->fresh + 1;
        const int ns = s->n_scale;
        if (ns < scale_frames) {
            s->scale[ns] = page;
            s->n_scale = ns + 1;
        } else {
            s->win[(head + n_win) % kMaxPool] = page;
            ++n_win;
        }
        s->n_sp = s->n_sp + nsp;
    }
    while (n_win > sliding_window) {
        s->free_[n_free++] = s->win[head];
        head = (head + 1) % kMaxPool;
        --n_win;
    }
    s->n_win = n_win;
    s->win_head = head;
    s->n_free = n_free;
}

// Discards the last appended frame: its K/V stay in the tentative slot and are
// never kept.
__global__ void k_rollback(CacheState* states, int count) {
    int c = blockIdx.x;
    if (c < count && threadIdx.x == 0) states[c].pending = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
    size_t n16 = bytes / 16;
    size_t ntail = bytes - n16 * 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)p, n16,
                       (unsigned char*)p + n16 * 16, ntail);
    return hipGetLastError();
}

hipError_t launch_reset(CacheState* states, int count, hipStream_t st) {
    hipLaunchKernelGGL(k_reset, dim3(count), dim3(64), 0, st, states, count);
    return hipGetLastError();
}

hipError_t launch_evict(CacheState* states, int count, int scale_frames, int sliding_window,
                        int max_sp_tokens, int nsp, hipStream_t st) {
    hipLaunchKernelGGL(k_evict, dim3(count), dim3(64), 0, st, states, count, scale_frames,
                       sliding_window, max_sp_tokens, nsp);
    return hipGetLastError();
}

hipError_t launch_rollback(CacheState* states, int count, hipStream_t st) {
    hipLaunchKernelGGL(k_rollback, dim3(count), dim3(64), 0, st, states, count);
    return hipGetLastError();
}

}  // namespace rpkv
