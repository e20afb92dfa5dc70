/*
 * rpkv.h -- C ABI of the per-frame hot path of a streaming 3D-reconstruction
 * transformer on AMD Instinct MI355X (gfx950):
 *
 *   3D (t/h/w) rotary embedding of the new frame's Q and K
 *     -> append of rotated K and raw V into a dual-stream paged KV cache
 *     -> attention of the frame's tokens over the retained pages
 *     -> deferred eviction of the oldest window page.
 *
 * Sources (web pages on the LingBot-Map streaming model):
 *   [ROPE-KV] "How 3D RoPE Positional Encoding Works with the Paged KV Cache in
 *             LingBot-Map"
 *   [VROPE]   "Video RoPE Positional Encoding: 3D Rotary Embeddings for
 *             Long-Sequence Video in Ling-Bot-Map"
 *   [RT3D]    "How LingBot-Map Achieves Real-Time 3D Reconstruction: Streaming
 *             Transformers and KV Caching"
 *   [LONG]    "How to Handle Sequences Exceeding the RoPE Training Range in
 *             LingBot-Map"
 *   [KVB]     "KV Caching Benefits in Ling Bot-Map: 7 Advantages for Streaming
 *             Vision Models"
 *
 * General conventions
 * -------------------
 * - Every function returns an int status: RPKV_OK (0) or a negative error
 *   code; nothing throws across the ABI.  rpkv_strerror() names a code.
 * - Device pointers are plain addresses of GPU memory owned by the caller
 *   (for instance the storage of torch tensors); the library never frees them.
 *   The library owns only the opaque host-side kv_handle.
 * - `stream` is a hipStream_t passed as void*.  Calls only enqueue work on
 *   that stream and return; none blocks the host except kv_read_state and
 *   rope3d_build_tables (which waits for its host->device copy).  The per-frame
 *   sequence kv_append_frame -> attend_frame -> kv_evict_deferred reads and
 *   writes cache bookkeeping only on the device, so it needs no host<->device
 *   synchronisation ([VROPE] "Cache-Friendly Pre-computation": no host sync on
 *   the streaming path).  One handle is used by one host thread and one stream
 *   at a time.
 * - Activations q, k, v, q_rot, out are row-major [S][N][H][D] with
 *   S = num_streams, N = special_tokens + grid_h*grid_w tokens per frame
 *   (the special tokens first, then the patches row by row: [ROPE-KV]
 *   "Multi-Axis Frequency Generation", patch_start_idx), H = num_heads,
 *   D = head_dim, in the cache dtype (bf16 or fp32), 16-byte aligned.
 * - Errors found on the device (cache pool or special stream exhausted) set a
 *   sticky per-cache status (read with kv_read_state); later appends of that
 *   cache write nothing to the cache and leave its visible set empty until
 *   kv_reset.  Attention over an empty visible set writes zeros and lse -inf.
 */
#ifndef RPKV_H
#define RPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    RPKV_OK = 0,
    RPKV_EINVAL = -1,   /* bad argument, shape, alignment or layer index */
    RPKV_EHIP = -2,     /* a HIP runtime call failed */
    RPKV_ENOSPACE = -3, /* patch pool or special stream exhausted (device status) */
    RPKV_ESTATE = -4,   /* call not valid in the handle's current state */
    RPKV_ETOOBIG = -5   /* request larger than the library's static scratch */
};

enum { RPKV_BF16 = 0, RPKV_F32 = 1 };

/* Maximum patch pool pages per cache (scale_frames + sliding_window + 1). */
#define RPKV_MAX_POOL_PAGES 512

/*
 * 3D rotary tables ([ROPE-KV] "Multi-Axis Frequency Generation"; [VROPE]
 * "The Three Rotary Dimensions", "NTK-Aware Frequency Scaling").
 *
 * The head's D/2 complex pairs (x[2j], x[2j+1]) are split into pairs_t, pairs_h,
 * pairs_w consecutive pairs for the frame (t), row (h) and column (w) axes.
 * Axis a with d_a = 2*pairs_a channels rotates pair j by pos_a * omega_{a,j},
 * omega_{a,j} = (theta*ntk_factor)^(-2j/d_a).  Token positions: specials of
 * frame f at (f, 0, 0), patch (r, c) at (f, r, c).
 *
 * Table layout in device memory (fp32, computed in fp64 on the host and
 * rounded once): three tables of (cos, sin) float pairs, back to back,
 *   T[max_frames][pairs_t], Hh[max_h][pairs_h], Ww[max_w][pairs_w].
 * The tables are sized from the grid (token counts), not from data, so no
 * device value is ever read back ([LONG] "Deriving Size from Token Count").
 */
/* Channel layout of the rotation (rope3d_spec.layout):
 *  - RPKV_ROPE_INTERLEAVED: pair j is channels (2j, 2j+1); the t axis takes
 *    pairs 0..pairs_t-1, then h, then w ([ROPE-KV] "Complex-Valued Tensor
 *    Application": a complex table of head_dim/2 entries per token);
 *  - RPKV_ROPE_HALF_SPLIT: axis a owns a block of 2*pairs_a consecutive
 *    channels (t, then h, then w) and pair i of that block is channels
 *    (b + i, b + i + pairs_a): the block is split in halves, the 2D module's
 *    arrangement ([LONG] "Understanding the 2D RoPE Architecture": vertical
 *    and horizontal halves, base frequency 100).  Every pairs_a must be a
 *    multiple of 8 here (whole 16-byte chunks per half). */
#define RPKV_ROPE_INTERLEAVED 0
#define RPKV_ROPE_HALF_SPLIT 1

typedef struct {
    int head_dim;       /* D, even; pairs_t + pairs_h + pairs_w == D/2 */
    int pairs_t, pairs_h, pairs_w;
    double theta;       /* base, e.g. 10000 (100 for the 2D module) */
    double ntk_factor;  /* multiplies theta; 1 = none */
    int max_frames;     /* rows of the t table: frame indices 0..max_frames-1 */
    int max_h, max_w;   /* rows of the h and w tables (>= grid_h, grid_w) */
    int layout;         /* RPKV_ROPE_INTERLEAVED or RPKV_ROPE_HALF_SPLIT */
} rope3d_spec;

/* Bytes of the rotary tables for `spec`; 0 if the spec is invalid. */
size_t rope3d_tables_bytes(const rope3d_spec* spec);

/* Computes the tables on the host (fp64 -> fp32) and copies them into the
 * caller's device buffer `d_tables` (>= rope3d_tables_bytes bytes) on `stream`,
 * waiting for the copy.  EINVAL on a bad spec or a short buffer. */
int rope3d_build_tables(const rope3d_spec* spec, void* d_tables, size_t bytes, void* stream);

/*
 * Dual-stream paged KV cache ([ROPE-KV] "Dual-Stream Memory Layout"):
 *  - patch stream: one page per stored frame (grid_h*grid_w patch tokens);
 *    the first scale_frames stored pages are permanent, the next form a
 *    sliding window of sliding_window pages whose oldest page returns to a
 *    free list (last in, first out) at kv_evict_deferred; pool =
 *    scale_frames + sliding_window + 1 pages per cache;
 *  - special stream: append-only, special_tokens tokens per stored frame in
 *    pages of special_page_size tokens, never evicted; capacity
 *    max_keyframes stored frames (+1 frame of tentative tokens).
 * One cache per (layer, stream).  Every appended frame first lands in the
 * tentative slot (the page the next stored frame takes and the special tokens
 * right after the stored ones); its own attention sees it there.  The deferred
 * eviction call then keeps it if it is a keyframe (commit = 1) -- the page
 * joins the scale list or the window, its specials the special stream -- and a
 * skip-append frame (commit = 0, [KVB] "Reduced KV Growth via Keyframe
 * Streaming") or a rolled-back one is simply not kept ([KVB] "Dynamic Keyframe
 * Selection": deferred eviction retains the KV, rollback drops it).
 *
 * Device memory (all inside the caller's d_mem, laid out by the library):
 *  - per cache: bookkeeping state (int32) and the visible page table;
 *  - K patch pool [layer][stream][head][page][slot][D] (row-major K),
 *    slot capacity = patch_page_size rounded up to 64;
 *  - V patch pool [layer][stream][head][page][D][slot] (V transposed per page;
 *    within every aligned group of 16 slots the storage order is slots 0-3,
 *    8-11, 4-7, 12-15, the order the attention kernel's matrix-core operands use);
 *  - K / V special streams [layer][stream][head][token][D] and
 *    [layer][stream][head][D][token] (same 16-slot order), token capacity
 *    rounded up to 64;
 *  - attention split scratch (partial outputs).
 * Padding: kv_create zero-fills everything.  An append zeroes the V^T padding
 * of the 64-slot tiles it writes; the K padding, and V^T tiles past the
 * frame's last tile, keep what they held, so a page recycled for a frame of a
 * smaller grid may hold an older frame's rows there.  Attention masks every
 * slot past a page's token count, so such rows never reach the softmax.
 */
typedef struct {
    int num_layers;         /* caches per stream (one per attention layer) */
    int num_streams;        /* independent streams batched in every call */
    int num_heads;          /* H */
    int head_dim;           /* D (64 for the bf16 matrix-core path) */
    int dtype;              /* RPKV_BF16 or RPKV_F32 */
    int grid_h, grid_w;     /* patch grid of a frame */
    int special_tokens;     /* special tokens per frame (6), <= 64 */
    int patch_page_size;    /* tokens per patch page, >= grid_h*grid_w */
    int special_page_size;  /* tokens per special page (6) */
    int scale_frames;       /* permanent patch pages */
    int sliding_window;     /* window pages kept after eviction */
    int max_keyframes;      /* stored frames the special stream can hold */
    int attn_splits;        /* key-range splits of attend_frame; 0 = automatic */
    rope3d_spec rope;       /* spec the caller's rotary tables were built with */
} kv_config;

typedef struct kv_handle kv_handle;

/* Bytes of device memory kv_create needs for `cfg`; 0 if cfg is invalid.
 * Besides the field limits above, a bf16 cache is invalid when one head's
 * patch pool or special stream would reach 4 GiB (the attention kernel
 * addresses a head through 32-bit buffer offsets). */
size_t kv_required_bytes(const kv_config* cfg);

/* Lays the cache out in the caller's d_mem (>= kv_required_bytes, 256-byte
 * aligned), zero-fills it on `stream` and returns a handle
 * ([ROPE-KV] "Implementation Example": FlashInferKVCacheManager(...)). */
int kv_create(const kv_config* cfg, void* d_mem, size_t bytes, void* stream, kv_handle** out);

/* Frees the host handle; the device memory stays the caller's. */
int kv_destroy(kv_handle* h);

/* Empties the caches of `layer` (-1: all layers) on the device: bookkeeping
 * back to its initial state, status cleared ([KVB] "Cross-Window Alignment for
 * Long Videos": clean_kv_cache). */
int kv_reset(kv_handle* h, int layer, void* stream);

/*
 * RoPE + append for one frame of every stream of `layer` ([ROPE-KV] "Frame
 * Appending and Position Encoding Integration"; [VROPE] "Temporal Consistency
 * in KV-Cache Streaming"; [KVB] "Reduced KV Growth via Keyframe Streaming").
 *   frame_idx: global frame index = temporal position t (0 <= t < rope.max_frames)
 *   commit:    1 keyframe (stored), 0 skip-append (tentative slot only)
 *   q, k, v:   inputs [S][N][H][D]; read only
 *   q_rot:     output [S][N][H][D]: rotated Q for attend_frame
 *   d_tables:  rotary tables built with cfg.rope
 * Rotated K and raw V go to the tentative slot; the visible page table is
 * rebuilt on the device: scale pages, window pages oldest first, the frame's
 * own page, then the special pages with their last-page length ([ROPE-KV]
 * "Attention Computation with Cached RoPE").  `commit` is recorded and applied
 * by kv_evict_deferred.  A second append without kv_evict_deferred or
 * kv_rollback in between replaces the first (same tentative slot).
 * No bookkeeping is read back to the host.
 */
int kv_append_frame(kv_handle* h, int layer, int frame_idx, int commit, const void* q,
                    const void* k, const void* v, void* q_rot, const void* d_tables,
                    void* stream);

/*
 * kv_append_frame for a frame of its own patch grid (grid_h x grid_w, at
 * most the configured grid_h*grid_w patches, grid_h <= rope.max_h and
 * grid_w <= rope.max_w): the cache takes variable patch counts per frame
 * ([ROPE-KV] FAQ on variable numbers of patches per frame: pages hold the
 * valid tokens they were given, attention reads those only).
 *   q, k, v, q_rot keep the [S][N][H][D] shape of the configuration; only
 *   the frame's first special_tokens + grid_h*grid_w tokens are read, and
 *   only those rows of q_rot are written.  Patch token p sits at
 *   (frame_idx, p / grid_w, p % grid_w).
 * The page records its token count; attend_frame then attends over the valid
 * tokens of every visible page and answers this frame's tokens only (rows
 * past them in out / lse are left as they were).  kv_append_frame is this
 * call with the configured grid.  EINVAL on a grid outside those bounds.
 */
int kv_append_frame_grid(kv_handle* h, int layer, int frame_idx, int commit, int grid_h,
                         int grid_w, const void* q, const void* k, const void* v, void* q_rot,
                         const void* d_tables, void* stream);

/*
 * QKV projection fused with RoPE + append, bf16 caches only: the rotary
 * embedding follows the Q/K projection and precedes the cache write
 * ([ROPE-KV] FAQ on where RoPE is applied relative to the KV cache write).
 * For every stream s, [Q | K | V] = x[s] w^T with fp32 accumulation, each
 * product rounded once to bf16; then exactly kv_append_frame(h, layer,
 * frame_idx, commit, Q, K, V, q_rot, d_tables) with the configured grid
 * (same rounding, target page, frame record and pending commit), without
 * Q, K and V ever being written to memory.
 *   x:      [S][N][hidden] bf16, the frame's hidden states; read only
 *   hidden: reduction length C, a multiple of 64 (>= 64)
 *   w:      [3*H*D][hidden] bf16, the layer's projection as a linear layer
 *           stores it (output channel major): rows 0 .. H*D-1 give Q (head h
 *           at rows h*D ..), then K, then V; no bias; read only
 *   q_rot:  output [S][N][H][D] bf16, as for kv_append_frame
 * EINVAL for an fp32 cache, an odd num_heads, a hidden size that is not a
 * positive multiple of 64, or a pointer that is null or not 16-byte aligned.
 */
int kv_project_append_frame(kv_handle* h, int layer, int frame_idx, int commit, const void* x,
                            int hidden, const void* w, void* q_rot, const void* d_tables,
                            void* stream);

/*
 * kv_project_append_frame for a frame of its own patch grid, exactly as
 * kv_append_frame_grid is kv_append_frame for one ([ROPE-KV] FAQ on variable
 * numbers of patches per frame): x keeps its [S][N][hidden] shape, only the
 * frame's first special_tokens + grid_h*grid_w rows are read, and only those
 * rows of q_rot are written; the page records its token count.  EINVAL on a
 * grid outside the bounds kv_append_frame_grid accepts, and as above.
 */
int kv_project_append_frame_grid(kv_handle* h, int layer, int frame_idx, int commit, int grid_h,
                                 int grid_w, const void* x, int hidden, const void* w, void* q_rot,
                                 const void* d_tables, void* stream);

/*
 * Attention of the frame's N query tokens (all heads, all streams) over the
 * visible page table of `layer` ([ROPE-KV] "Attention Computation with Cached
 * RoPE"; [RT3D] "Per-Frame Processing and Causal Attention"):
 *   out[s][i][h][:] = sum_j softmax_j(q_rot[s][i][h]·K_j / sqrt(D)) V_j over
 *   every visible token j (no mask inside the visible set).
 *   q_rot: [S][N][H][D]; out: [S][N][H][D] in the cache dtype;
 *   lse:   optional [S][H][N] fp32 natural-log log-sum-exp of the scaled
 *          scores (NULL to skip).
 * bf16 runs on the matrix cores (bf16 products, fp32 accumulation, online
 * softmax); fp32 runs in fp32 throughout.
 */
int attend_frame(kv_handle* h, int layer, const void* q_rot, void* out, float* lse, void* stream);

/*
 * attend_frame for callers that cannot allocate device memory or take a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, kernels and results as
 * attend_frame (bit for bit); the split partial outputs go to a static array
 * inside the library instead of the handle's memory, and the call allocates
 * nothing.  Limit: a handle whose split scratch, S*H*splits*N*136 bytes
 * (rounded up), exceeds RPKV_STATIC_SCRATCH_BYTES gets RPKV_ETOOBIG; with one
 * split nothing is used.  The array is per GPU, held by every process that
 * loads the library until it ends, and shared by every call on that GPU:
 * calls that may run at the same time on one GPU (other streams, other
 * threads) race on it and must be ordered by the caller.
 */
#define RPKV_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int attend_frame_noalloc(kv_handle* h, int layer, const void* q_rot, void* out, float* lse,
                         void* stream);

/*
 * Residual update after an attention layer, fused with the cast feeding the
 * next layer's projection (page "How LingBot-Map Achieves Real-Time 3D
 * Reconstruction", section "AggregatorStream with FlashInfer Paged KV Cache":
 * each frame and global block adds its attention output back into the token
 * stream).  For i in [0, n):
 *   x[i]  <- x[i] + o[i]       in fp32 (o widened exactly, one rounding)
 *   xb[i] <- x[i] rounded to bf16, nearest even (NaN stays NaN)
 *   x:  fp32, read and written;  o: bf16 bits, read only (attend_frame's out
 *       viewed flat);  xb: bf16 bits, written, or NULL to skip the cast.
 * Elementwise, so any shape flattened to n elements; x, o and xb must not
 * overlap.  n = 0 launches nothing.  EINVAL for n < 0 or n >= 2^40, or a
 * pointer that is null (xb aside) or not 16-byte aligned.
 */
int residual_add_bf16(float* x, const void* o, void* xb, long long n, void* stream);

/* Deferred eviction for `layer` ([KVB] "Memory-Efficient Sliding Window
 * Management", "Dynamic Keyframe Selection"; [ROPE-KV] "Dual-Stream Memory
 * Layout"), run after the frame's attention: first keeps the last appended
 * frame if it was appended with commit = 1 (ENOSPACE, sticky, if the special
 * stream already holds max_keyframes frames), then, while a cache's window
 * holds more than sliding_window pages, moves its oldest page to the free list.
 * Policy parameters are the ones given at kv_create. */
int kv_evict_deferred(kv_handle* h, int layer, void* stream);

/* Drops the last appended frame of every stream of `layer` instead of keeping
 * it ([KVB] "Dynamic Keyframe Selection": _rollback_last_frame removes the
 * temporary KV entry).  Lets a caller decide keyframes after attention:
 * append with commit = 1, attend, then kv_evict_deferred (keep) or
 * kv_rollback (drop; a following kv_evict_deferred is a no-op). */
int kv_rollback(kv_handle* h, int layer, void* stream);

/* Bookkeeping of one cache, copied to the host (test and debug hook). */
typedef struct {
    int status;                 /* RPKV_OK or RPKV_ENOSPACE (sticky) */
    int fresh;                  /* never-used pages start here */
    int n_free, n_scale, n_window;
    int n_special_tokens;       /* committed special tokens */
    int target_page;            /* page written by the last append */
    int special_offset;         /* first special token written by the last append */
    int n_visible_pages;        /* patch pages in the visible table */
    int visible_special_pages;  /* special pages 0 .. visible_special_pages-1 */
    int last_page_len;          /* valid tokens in the last visible special page */
    int visible_special_tokens;
    int pending_commit;         /* 1: last appended keyframe not yet kept */
    int free_list[RPKV_MAX_POOL_PAGES];    /* bottom .. top */
    int scale_pages[RPKV_MAX_POOL_PAGES];
    int window_pages[RPKV_MAX_POOL_PAGES]; /* oldest first */
    int visible_pages[RPKV_MAX_POOL_PAGES];
    int query_tokens;           /* tokens of the last appended frame */
    int page_tokens[RPKV_MAX_POOL_PAGES];  /* tokens stored in each pool page (0: never written) */
} kv_state_host;

/* Copies the state of cache (layer, stream_idx) after the work queued on
 * `stream`; waits for the stream. */
int kv_read_state(kv_handle* h, int layer, int stream_idx, kv_state_host* out, void* stream);

/* Static sizes of a handle plus host-side counters of the calls made
 * ([KVB] "Working with the KV Cache API": get_kv_cache_info).  Reads nothing
 * from the device. */
typedef struct {
    int num_layers, num_streams, num_heads, head_dim, dtype;
    int tokens_per_frame;       /* N */
    int pool_pages;             /* patch pages per cache */
    int slot_capacity;          /* padded tokens per patch page */
    int special_capacity;       /* padded special tokens per cache */
    int attn_splits;
    size_t page_bytes;          /* K + V bytes of one patch page, all heads */
    size_t cache_bytes;         /* K + V pools of one cache */
    size_t total_bytes;         /* kv_required_bytes */
    /* byte offsets inside d_mem of the K pool, V pool, K special stream and
     * V special stream (all layers and streams, layout above): inspection only */
    size_t off_kpool, off_vpool, off_ksp, off_vsp;
    long long frames_appended;  /* appends of layer 0 (every append entry point) since
                                   kv_create or the last kv_reset of layer 0 / all layers */
    long long frames_committed; /* layer-0 appends with commit = 1 that kv_evict_deferred
                                   then kept: not dropped by kv_rollback, not replaced by
                                   a second append.  Host-side count: a commit the device
                                   refuses (special stream full: sticky RPKV_ENOSPACE,
                                   seen with kv_read_state) is still counted */
} kv_info;

int kv_get_info(const kv_handle* h, kv_info* out);

const char* rpkv_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* RPKV_H */
