// Internal definitions shared by the HIP translation units of librpkv.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rpkv.h"

namespace rpkv {

constexpr int kHeadDim = 64;      // D: the kernels are written for 64-wide heads
constexpr int kTile = 64;         // keys per attention tile, slots per append tile
constexpr int kMaxPool = RPKV_MAX_POOL_PAGES;

// Bookkeeping of one (layer, stream) cache, resident in device memory.
// Structural fields (free list, scale list, window, counters) change only in
// the commit/eviction and reset kernels; the append kernel writes the frame
// record (target, sp_off, pending, visible table); every kernel reads.
struct CacheState {
    int pending;        // 1: the last appended frame is a keyframe not yet committed
    int status;         // RPKV_OK or RPKV_ENOSPACE (sticky)
    int fresh;          // never-used pages are fresh .. pool-1
    int n_free;         // free list (stack) size
    int n_scale;        // permanent pages
    int win_head;       // ring index of the oldest window page
    int n_win;          // window pages
    int n_sp;           // committed special tokens
    int target;         // page written by the last append
    int sp_off;         // first special token written by the last append
    int vis_n;          // patch pages in the visible table
    int vis_sp_pages;   // special pages 0 .. vis_sp_pages-1 visible
    int last_page_len;  // valid tokens in the last visible special page
    int vis_sp_tokens;  // visible special tokens
    int n_query;        // tokens of the last appended frame (specials + its patches)
    int vis_full;       // 1: every visible patch page holds a whole grid (P tokens)
    int free_[kMaxPool];
    int scale[kMaxPool];
    int win[kMaxPool];  // ring buffer of capacity kMaxPool
    int vis[kMaxPool];  // visible patch pages in attention order
    int vis_len[kMaxPool];      // tokens of each visible patch page
    int page_tokens[kMaxPool];  // tokens stored in each pool page (its frame's patches)
    // key tiles of the visible patch pages before page i (ceil(len / kTile)
    // each); [vis_n] is their total.  Written with the visible table, read
    // when vis_full is 0.
    int vis_tpre[kMaxPool + 1];
};

// Storage position <-> key index inside an aligned group of 16 slots of a
// transposed V page: positions 0-3, 4-7, 8-11, 12-15 hold keys 0-3, 8-11,
// 4-7, 12-15.  The map is its own inverse.
__host__ __device__ inline int vslot_perm(int p) {
    return (p & ~12) | (((p >> 2) & 1) << 3) | (((p >> 3) & 1) << 2);
}

struct Layout {
    int S, H, N, P, nsp, gh, gw;
    int pool, slot_cap, sp_cap, sp_page, sf, W, max_kf;
    int tpp;            // attention tiles per patch page
    int q_tiles;        // 128-query tiles per frame
    int splits;
    int elem;           // bytes per element
    size_t state_bytes; // per cache, padded
    size_t kpool_elems; // per cache (K; V has the same count)
    size_t ksp_elems;   // per cache
    // byte offsets inside the handle's device memory
    size_t off_state, off_kpool, off_vpool, off_ksp, off_vsp, off_part_o, off_part_ls, total;
};

struct AppendArgs {
    const void* q;
    const void* k;
    const void* v;
    void* q_rot;
    const float2* tab_t;
    const float2* tab_h;
    const float2* tab_w;
    CacheState* states;     // caches of this layer, one per stream
    char* kpool;            // this layer's K pool (stream s at s*kpool_elems)
    char* vpool;
    char* ksp;
    char* vsp;
    size_t kpool_elems, ksp_elems;
    int S, N, H, P, gw, nsp, pool, slot_cap, sp_cap, sp_page, sf, max_kf;
    int fP, fgw;            // this frame's patches (<= P) and its grid width
    int pt, ph, pw;
    int layout;             // RPKV_ROPE_INTERLEAVED or RPKV_ROPE_HALF_SPLIT
    int frame, commit;
    int n_tiles;            // workgroups per (stream, head)
};

// The fused projection + append: the append's arguments (q, k, v unused)
// plus the projection operands.
struct ProjArgs {
    AppendArgs a;
    const uint16_t* x;      // [S][N][C] bf16
    const uint16_t* w;      // [3*H*D][C] bf16
    int C;
    int row_blocks;         // 128-row tiles of the frame's tokens
    int col_blocks;         // 128-channel tiles of the 3*H*D outputs
};

struct AttnArgs {
    const void* q;          // q_rot [S][N][H][D]
    void* out;              // [S][N][H][D]
    float* lse;             // [S][H][N] or null
    const CacheState* states;
    const char* kpool;
    const char* vpool;
    const char* ksp;
    const char* vsp;
    size_t kpool_elems, ksp_elems;
    uint16_t* part_o;       // [S][H][splits][N][D], fp16 bits, each row scaled by 2^-e
    float2* part_ls;        // [S][H][splits][N]: (LSE, factor 2^e / l of the row)
    int S, N, H, P, pool, slot_cap, sp_cap, tpp, splits, q_tiles;
    int n_logical;          // workgroups doing work (grid may be padded)
    float scale;            // 1/sqrt(D)
    float scale_log2;       // scale * log2(e)
};

// Launchers (one per translation unit).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_reset(CacheState* states, int count, hipStream_t st);
hipError_t launch_evict(CacheState* states, int count, int scale_frames, int sliding_window,
                        int max_sp_tokens, int nsp, hipStream_t st);
hipError_t launch_rollback(CacheState* states, int count, hipStream_t st);
hipError_t launch_rope_append(const AppendArgs& a, int dtype, hipStream_t st);
hipError_t launch_project_append(const ProjArgs& p, hipStream_t st);
hipError_t launch_attend(const AttnArgs& a, int dtype, hipStream_t st);
hipError_t launch_attend_bf16_main(const AttnArgs& a, hipStream_t st);
hipError_t launch_residual_add(float* x, const uint16_t* o, uint16_t* xb, long long n,
                               hipStream_t st);

}  // namespace rpkv
