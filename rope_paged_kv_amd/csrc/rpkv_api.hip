// Host side of the C ABI declared in include/rpkv.h: argument checks, the
// device-memory layout of a handle, rotary-table construction and kernel
// launches.  No call synchronises the host except rope3d_build_tables (its
// copy) and kv_read_state.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "rpkv_internal.h"

using namespace rpkv;

struct kv_handle {
    kv_config cfg;
    Layout L;
    char* base;
    size_t bytes;
    long long appended, committed;
    bool pending0;   // layer 0's last append asked to be kept and was neither kept nor dropped yet
};

namespace {

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool spec_ok(const rope3d_spec* r) {
    if (!r || r->head_dim <= 0 || r->head_dim % 2 || r->pairs_t < 0 || r->pairs_h < 0 || r->pairs_w < 0 ||
        r->pairs_t + r->pairs_h + r->pairs_w != r->head_dim / 2 || !(r->theta > 0) ||
        !(r->ntk_factor > 0) || r->max_frames < 1 || r->max_h < 1 || r->max_w < 1)
        return false;
    if (r->layout == RPKV_ROPE_HALF_SPLIT)
        return r->pairs_t % 8 == 0 && r->pairs_h % 8 == 0 && r->pairs_w % 8 == 0;
    return r->layout == RPKV_ROPE_INTERLEAVED;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Key-range splits of attend_frame.  The bf16 kernel is bound by what each
// compute unit (256 on MI355X) issues, so a launch lasts about as long as
// the most loaded unit needs for its ceil(workgroups / 256) workgroups, and
// with fewer than 2 workgroups per unit it runs ~1.5x slower per workgroup;
// splitting shortens each workgroup but adds a round trip of partial
// outputs through the merge (per query, head and split: 64 fp16 channels
// plus the fp32 LSE and row factor, written and read back: 272 bytes).  The
// estimate (microseconds, from measured
// rates: ~0.55 us per 64-key tile of a workgroup on a busy unit, ~2 tiles of
// fixed cost per workgroup, partials moved at ~4 TB/s, ~3 us per merge
// launch) is taken at the largest visible set the cache can hold.
int auto_splits(const Layout& L) {
    constexpr int kCUs = 256;
    const long long base = (long long)L.q_tiles * L.H * L.S;
    const int max_tiles = L.pool * L.tpp + (L.sp_cap + kTile - 1) / kTile;
    const double part_us = (double)L.S * L.H * L.N * 272.0 / 4.0e6;
    int best = 1;
    double best_us = 0.0;
    for (int s = 1; s <= 32 && s <= max_tiles; ++s) {
        const long long wg = base * s;
        const double busy = (double)((wg + kCUs - 1) / kCUs) * ((double)max_tiles / s + 2.0) * 0.552;
        const double us = busy * (wg < 2 * kCUs ? 1.5 : 1.0) + (s > 1 ? 3.0 + s * part_us : 0.0);
        if (s == 1 || us < best_us) {
            best = s;
            best_us = us;
        }
    }
    return best;
}

bool layout(const kv_config* c, Layout* L) {
    if (!c) return false;
    if (c->num_layers < 1 || c->num_streams < 1 || c->num_heads < 1 || c->head_dim != kHeadDim)
        return false;
    if (c->dtype != RPKV_BF16 && c->dtype != RPKV_F32) return false;
    if (c->grid_h < 1 || c->grid_w < 1 || c->special_tokens < 0 || c->special_tokens > kTile)
        return false;
    const long long P = (long long)c->grid_h * c->grid_w;
    if (P > (1 << 20) || c->patch_page_size < P || c->special_page_size < 1) return false;
    if (c->scale_frames < 0 || c->sliding_window < 0 ||
        c->scale_frames + c->sliding_window + 1 > kMaxPool)
        return false;
    if (c->max_keyframes < 0 || c->attn_splits < 0) return false;
    if (!spec_ok(&c->rope) || c->rope.head_dim != c->head_dim || c->rope.max_h < c->grid_h ||
        c->rope.max_w < c->grid_w)
        return false;
    Layout& l = *L;
    l.S = c->num_streams;
    l.H = c->num_heads;
    l.P = (int)P;
    l.nsp = c->special_tokens;
    l.N = l.nsp + l.P;
    l.gh = c->grid_h;
    l.gw = c->grid_w;
    l.pool = c->scale_frames + c->sliding_window + 1;
    l.slot_cap = (int)round_up((size_t)c->patch_page_size, kTile);
    l.sp_page = c->special_page_size;
    // committed specials + one tentative frame, whole special pages, 64-aligned
    const size_t sp_tok = (size_t)(c->max_keyframes + 1) * c->special_tokens;
    const size_t sp_pages_tok = round_up(sp_tok, (size_t)c->special_page_size);
    l.sp_cap = (int)round_up(sp_pages_tok > 0 ? sp_pages_tok : 1, kTile);
    l.sf = c->scale_frames;
    l.W = c->sliding_window;
    l.max_kf = c->max_keyframes;
    l.tpp = (l.P + kTile - 1) / kTile;
    l.q_tiles = (l.N + 127) / 128;
    l.elem = c->dtype == RPKV_BF16 ? 2 : 4;
    if (c->dtype == RPKV_F32)
        l.splits = 1;
    else
        l.splits = c->attn_splits > 0 ? (c->attn_splits > 64 ? 64 : c->attn_splits) : auto_splits(l);
    // The bf16 attention kernel addresses one head's pages through a 32-bit
    // buffer offset.
    if (c->dtype == RPKV_BF16 && ((size_t)l.pool * l.slot_cap * kHeadDim * 2 >= (1ull << 32) ||
                                  (size_t)l.sp_cap * kHeadDim * 2 >= (1ull << 32)))
        return false;
    l.state_bytes = round_up(sizeof(CacheState), 256);
    l.kpool_elems = (size_t)l.H * l.pool * l.slot_cap * kHeadDim;
    l.ksp_elems = (size_t)l.H * l.sp_cap * kHeadDim;
    const size_t caches = (size_t)c->num_layers * l.S;
    l.off_state = 0;
    l.off_kpool = round_up(caches * l.state_bytes, 256);
    l.off_vpool = l.off_kpool + round_up(caches * l.kpool_elems * l.elem, 256);
    l.off_ksp = l.off_vpool + round_up(caches * l.kpool_elems * l.elem, 256);
    l.off_vsp = l.off_ksp + round_up(caches * l.ksp_elems * l.elem, 256);
    l.off_part_o = l.off_vsp + round_up(caches * l.ksp_elems * l.elem, 256);
    const size_t parts = l.splits > 1 ? (size_t)l.S * l.H * l.splits * l.N : 0;
    l.off_part_ls = l.off_part_o + round_up(parts * kHeadDim * 2, 256);   // fp16 words
    l.total = l.off_part_ls + round_up(parts * 8, 256);                   // (LSE, factor)
    return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? RPKV_OK : RPKV_EHIP; }

// Split scratch of attend_frame_noalloc, for callers that cannot allocate:
// the partial outputs and their (LSE, factor) pairs live in this array
// instead of the handle's memory.  Every GPU the library runs on holds its own
// copy until the process ends.  Host code never passes the array's name to a
// kernel (on the host it stands for a host-side shadow, not a device address):
// the device address is looked up once per device, with that device current,
// and kept in scratch_ptr.  Every call on a GPU shares that GPU's copy, so
// calls that overlap on one GPU race.  Nothing in it needs clearing: each
// call writes every row its merge reads.
static __device__ __align__(256) char scratch[RPKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char* scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (resolved on first use).
hipError_t current_scratch(char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = (char*)p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

// Bytes of split scratch one attend_frame call of this layout uses: fp16
// partial outputs, then (LSE, factor) pairs.
size_t split_scratch_bytes(const Layout& L, size_t* off_ls) {
    const size_t parts = L.splits > 1 ? (size_t)L.S * L.H * L.splits * L.N : 0;
    *off_ls = round_up(parts * kHeadDim * 2, 256);
    return *off_ls + round_up(parts * 8, 256);
}

CacheState* states_of(kv_handle* h, int layer) {
    return (CacheState*)(h->base + h->L.off_state) + (size_t)layer * h->L.S;
}

}  // namespace

extern "C" {

size_t rope3d_tables_bytes(const rope3d_spec* s) {
    if (!spec_ok(s)) return 0;
    return ((size_t)s->max_frames * s->pairs_t + (size_t)s->max_h * s->pairs_h +
            (size_t)s->max_w * s->pairs_w) * 2 * sizeof(float);
}

// Per-axis tables of (cos, sin)(pos * omega_j), omega_j = (theta*ntk)^(-2j/d_a),
// d_a = 2*pairs_a, computed in double and rounded once to float.
int rope3d_build_tables(const rope3d_spec* s, void* d_tables, size_t bytes, void* stream) {
    const size_t need = rope3d_tables_bytes(s);
    if (!need || !d_tables || bytes < need) return RPKV_EINVAL;
    float* host = (float*)malloc(need);
    if (!host) return RPKV_EINVAL;
    const double base = s->theta * s->ntk_factor;
    const int rows[3] = {s->max_frames, s->max_h, s->max_w};
    const int pairs[3] = {s->pairs_t, s->pairs_h, s->pairs_w};
    size_t o = 0;
    for (int ax = 0; ax < 3; ++ax) {
        const int np = pairs[ax];
        for (int pos = 0; pos < rows[ax]; ++pos)
            for (int j = 0; j < np; ++j) {
                const double omega = pow(base, -2.0 * j / (2.0 * np));
                const double ang = (double)pos * omega;
                host[o++] = (float)cos(ang);
                host[o++] = (float)sin(ang);
            }
    }
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(d_tables, host, need, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    free(host);
    return hip_status(e);
}

size_t kv_required_bytes(const kv_config* cfg) {
    Layout L;
    return layout(cfg, &L) ? L.total : 0;
}

int kv_create(const kv_config* cfg, void* d_mem, size_t bytes, void* stream, kv_handle** out) {
    if (!out) return RPKV_EINVAL;
    *out = nullptr;
    Layout L;
    if (!layout(cfg, &L) || !d_mem || ((uintptr_t)d_mem & 255) || bytes < L.total) return RPKV_EINVAL;
    kv_handle* h = new (std::nothrow) kv_handle;
    if (!h) return RPKV_EINVAL;
    h->cfg = *cfg;
    h->L = L;
    h->base = (char*)d_mem;
    h->bytes = bytes;
    h->appended = h->committed = 0;
    h->pending0 = false;
    hipStream_t st = (hipStream_t)stream;
    // Library set-up on this device: the static split scratch's address.
    char* scr = nullptr;
    hipError_t e = current_scratch(&scr);
    if (e == hipSuccess) e = launch_fill_zero(d_mem, L.total, st);
    if (e == hipSuccess) e = launch_reset(states_of(h, 0), cfg->num_layers * L.S, st);
    if (e != hipSuccess) {
        delete h;
        return RPKV_EHIP;
    }
    *out = h;
    return RPKV_OK;
}

int kv_destroy(kv_handle* h) {
    delete h;
    return RPKV_OK;
}

int kv_reset(kv_handle* h, int layer, void* stream) {
    if (!h || layer < -1 || layer >= h->cfg.num_layers) return RPKV_EINVAL;
    const int first = layer < 0 ? 0 : layer;
    const int count = (layer < 0 ? h->cfg.num_layers : 1) * h->L.S;
    if (layer <= 0) {
        h->appended = h->committed = 0;
        h->pending0 = false;
    }
    return hip_status(launch_reset(states_of(h, first), count, (hipStream_t)stream));
}

int kv_append_frame(kv_handle* h, int layer, int frame_idx, int commit, const void* q,
                    const void* k, const void* v, void* q_rot, const void* d_tables,
                    void* stream) {
    if (!h) return RPKV_EINVAL;
    return kv_append_frame_grid(h, layer, frame_idx, commit, h->cfg.grid_h, h->cfg.grid_w, q, k, v,
                                q_rot, d_tables, stream);
}

// Append arguments of one frame of `layer` (shared by the plain and the fused
// append).
static AppendArgs append_args(kv_handle* h, int layer, int frame_idx, int commit, int grid_h,
                              int grid_w, const void* q, const void* k, const void* v,
                              void* q_rot, const void* d_tables) {
    const Layout& L = h->L;
    const rope3d_spec& r = h->cfg.rope;
    AppendArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.q_rot = q_rot;
    a.tab_t = (const float2*)d_tables;
    a.tab_h = a.tab_t + (size_t)r.max_frames * r.pairs_t;
    a.tab_w = a.tab_h + (size_t)r.max_h * r.pairs_h;
    a.states = states_of(h, layer);
    const size_t caches_before = (size_t)layer * L.S;
    a.kpool = h->base + L.off_kpool + caches_before * L.kpool_elems * L.elem;
    a.vpool = h->base + L.off_vpool + caches_before * L.kpool_elems * L.elem;
    a.ksp = h->base + L.off_ksp + caches_before * L.ksp_elems * L.elem;
    a.vsp = h->base + L.off_vsp + caches_before * L.ksp_elems * L.elem;
    a.kpool_elems = L.kpool_elems;
    a.ksp_elems = L.ksp_elems;
    a.S = L.S;
    a.N = L.N;
    a.H = L.H;
    a.P = L.P;
    a.gw = L.gw;
    a.fP = grid_h * grid_w;
    a.fgw = grid_w;
    a.nsp = L.nsp;
    a.pool = L.pool;
    a.slot_cap = L.slot_cap;
    a.sp_cap = L.sp_cap;
    a.sp_page = L.sp_page;
    a.sf = L.sf;
    a.max_kf = L.max_kf;
    a.pt = r.pairs_t;
    a.ph = r.pairs_h;
    a.pw = r.pairs_w;
    a.layout = r.layout;
    a.frame = frame_idx;
    a.commit = commit;
    a.n_tiles = 1 + L.tpp;
    return a;
}

int kv_append_frame_grid(kv_handle* h, int layer, int frame_idx, int commit, int grid_h,
                         int grid_w, const void* q, const void* k, const void* v, void* q_rot,
                         const void* d_tables, void* stream) {
    if (!h || layer < 0 || layer >= h->cfg.num_layers) return RPKV_EINVAL;
    if (frame_idx < 0 || frame_idx >= h->cfg.rope.max_frames || (commit != 0 && commit != 1))
        return RPKV_EINVAL;
    if (grid_h < 1 || grid_w < 1 || grid_h > h->cfg.rope.max_h || grid_w > h->cfg.rope.max_w ||
        (long long)grid_h * grid_w > h->L.P)
        return RPKV_EINVAL;
    if (!q || !k || !v || !q_rot || !d_tables) return RPKV_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_rot) || !aligned16(d_tables))
        return RPKV_EINVAL;
    AppendArgs a = append_args(h, layer, frame_idx, commit, grid_h, grid_w, q, k, v, q_rot, d_tables);
    const int rc = hip_status(launch_rope_append(a, h->cfg.dtype, (hipStream_t)stream));
    if (rc == RPKV_OK && layer == 0) {
        h->appended++;
        h->pending0 = commit != 0;   // replaces an append not yet kept or dropped
    }
    return rc;
}

int kv_project_append_frame(kv_handle* h, int layer, int frame_idx, int commit, const void* x,
                            int hidden, const void* w, void* q_rot, const void* d_tables,
                            void* stream) {
    if (!h) return RPKV_EINVAL;
    return kv_project_append_frame_grid(h, layer, frame_idx, commit, h->cfg.grid_h, h->cfg.grid_w, x,
                                        hidden, w, q_rot, d_tables, stream);
}

int kv_project_append_frame_grid(kv_handle* h, int layer, int frame_idx, int commit, int grid_h,
                                 int grid_w, const void* x, int hidden, const void* w, void* q_rot,
                                 const void* d_tables, void* stream) {
    if (!h || layer < 0 || layer >= h->cfg.num_layers) return RPKV_EINVAL;
    if (grid_h < 1 || grid_w < 1 || grid_h > h->cfg.rope.max_h || grid_w > h->cfg.rope.max_w ||
        (long long)grid_h * grid_w > h->L.P)
        return RPKV_EINVAL;
    if (h->cfg.dtype != RPKV_BF16 || h->L.H % 2 != 0) return RPKV_EINVAL;
    if (frame_idx < 0 || frame_idx >= h->cfg.rope.max_frames || (commit != 0 && commit != 1))
        return RPKV_EINVAL;
    if (hidden < 64 || hidden % 64 != 0) return RPKV_EINVAL;
    if (!x || !w || !q_rot || !d_tables) return RPKV_EINVAL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(q_rot) || !aligned16(d_tables)) return RPKV_EINVAL;
    ProjArgs p;
    p.a = append_args(h, layer, frame_idx, commit, grid_h, grid_w, nullptr, nullptr, nullptr, q_rot,
                      d_tables);
    p.x = (const uint16_t*)x;
    p.w = (const uint16_t*)w;
    p.C = hidden;
    p.row_blocks = (p.a.fP + p.a.nsp + 127) / 128;
    p.col_blocks = 3 * h->L.H * kHeadDim / 128;
    const int rc = hip_status(launch_project_append(p, (hipStream_t)stream));
    if (rc == RPKV_OK && layer == 0) {
        h->appended++;
        h->pending0 = commit != 0;
    }
    return rc;
}

// Attention arguments of one call; the split scratch is set by the caller.
static AttnArgs attend_args(kv_handle* h, int layer, const void* q_rot, void* out, float* lse) {
    const Layout& L = h->L;
    AttnArgs a;
    a.q = q_rot;
    a.out = out;
    a.lse = lse;
    a.states = states_of(h, layer);
    const size_t caches_before = (size_t)layer * L.S;
    a.kpool = h->base + L.off_kpool + caches_before * L.kpool_elems * L.elem;
    a.vpool = h->base + L.off_vpool + caches_before * L.kpool_elems * L.elem;
    a.ksp = h->base + L.off_ksp + caches_before * L.ksp_elems * L.elem;
    a.vsp = h->base + L.off_vsp + caches_before * L.ksp_elems * L.elem;
    a.kpool_elems = L.kpool_elems;
    a.ksp_elems = L.ksp_elems;
    a.S = L.S;
    a.N = L.N;
    a.H = L.H;
    a.P = L.P;
    a.pool = L.pool;
    a.slot_cap = L.slot_cap;
    a.sp_cap = L.sp_cap;
    a.tpp = L.tpp;
    a.splits = L.splits;
    a.q_tiles = L.q_tiles;
    a.n_logical = L.q_tiles * L.H * L.S * L.splits;
    a.scale = 1.0f / sqrtf((float)kHeadDim);
    a.scale_log2 = (float)(1.0 / sqrt((double)kHeadDim) * 1.4426950408889634);
    return a;
}

int attend_frame(kv_handle* h, int layer, const void* q_rot, void* out, float* lse, void* stream) {
    if (!h || layer < 0 || layer >= h->cfg.num_layers || !q_rot || !out) return RPKV_EINVAL;
    if (!aligned16(q_rot) || !aligned16(out) || ((uintptr_t)lse & 3)) return RPKV_EINVAL;
    AttnArgs a = attend_args(h, layer, q_rot, out, lse);
    a.part_o = (uint16_t*)(h->base + h->L.off_part_o);
    a.part_ls = (float2*)(h->base + h->L.off_part_ls);
    return hip_status(launch_attend(a, h->cfg.dtype, (hipStream_t)stream));
}

int attend_frame_noalloc(kv_handle* h, int layer, const void* q_rot, void* out, float* lse,
                         void* stream) {
    if (!h || layer < 0 || layer >= h->cfg.num_layers || !q_rot || !out) return RPKV_EINVAL;
    if (!aligned16(q_rot) || !aligned16(out) || ((uintptr_t)lse & 3)) return RPKV_EINVAL;
    size_t off_ls = 0;
    if (split_scratch_bytes(h->L, &off_ls) > RPKV_STATIC_SCRATCH_BYTES) return RPKV_ETOOBIG;
    char* scr = nullptr;
    if (current_scratch(&scr) != hipSuccess) return RPKV_EHIP;
    AttnArgs a = attend_args(h, layer, q_rot, out, lse);
    a.part_o = (uint16_t*)scr;
    a.part_ls = (float2*)(scr + off_ls);
    return hip_status(launch_attend(a, h->cfg.dtype, (hipStream_t)stream));
}

int residual_add_bf16(float* x, const void* o, void* xb, long long n, void* stream) {
    if (n < 0 || n >= (1LL << 40) || !x || !o) return RPKV_EINVAL;
    if (!aligned16(x) || !aligned16(o) || (xb && !aligned16(xb))) return RPKV_EINVAL;
    if (n == 0) return RPKV_OK;
    return hip_status(launch_residual_add(x, (const uint16_t*)o, (uint16_t*)xb, n, (hipStream_t)stream));
}

int kv_evict_deferred(kv_handle* h, int layer, void* stream) {
    if (!h || layer < 0 || layer >= h->cfg.num_layers) return RPKV_EINVAL;
    const Layout& L = h->L;
    const int rc = hip_status(launch_evict(states_of(h, layer), L.S, L.sf, L.W, L.max_kf * L.nsp,
                                           L.nsp, (hipStream_t)stream));
    if (rc == RPKV_OK && layer == 0 && h->pending0) {
        h->committed++;
        h->pending0 = false;
    }
    return rc;
}

int kv_rollback(kv_handle* h, int layer, void* stream) {
    if (!h || layer < 0 || layer >= h->cfg.num_layers) return RPKV_EINVAL;
    const int rc = hip_status(launch_rollback(states_of(h, layer), h->L.S, (hipStream_t)stream));
    if (rc == RPKV_OK && layer == 0) h->pending0 = false;
    return rc;
}

int kv_read_state(kv_handle* h, int layer, int stream_idx, kv_state_host* out, void* stream) {
    if (!h || !out || layer < 0 || layer >= h->cfg.num_layers || stream_idx < 0 ||
        stream_idx >= h->L.S)
        return RPKV_EINVAL;
    CacheState* tmp = (CacheState*)malloc(sizeof(CacheState));
    if (!tmp) return RPKV_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(tmp, states_of(h, layer) + stream_idx, sizeof(CacheState),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        free(tmp);
        return RPKV_EHIP;
    }
    memset(out, 0, sizeof(*out));
    out->status = tmp->status;
    out->fresh = tmp->fresh;
    out->n_free = tmp->n_free;
    out->n_scale = tmp->n_scale;
    out->n_window = tmp->n_win;
    out->n_special_tokens = tmp->n_sp;
    out->target_page = tmp->target;
    out->special_offset = tmp->sp_off;
    out->n_visible_pages = tmp->vis_n;
    out->visible_special_pages = tmp->vis_sp_pages;
    out->last_page_len = tmp->last_page_len;
    out->visible_special_tokens = tmp->vis_sp_tokens;
    out->pending_commit = tmp->pending;
    for (int i = 0; i < tmp->n_free && i < kMaxPool; ++i) out->free_list[i] = tmp->free_[i];
    for (int i = 0; i < tmp->n_scale && i < kMaxPool; ++i) out->scale_pages[i] = tmp->scale[i];
    for (int i = 0; i < tmp->n_win && i < kMaxPool; ++i)
        out->window_pages[i] = tmp->win[(tmp->win_head + i) % kMaxPool];
    for (int i = 0; i < tmp->vis_n && i < kMaxPool; ++i) out->visible_pages[i] = tmp->vis[i];
    out->query_tokens = tmp->n_query;
    for (int i = 0; i < h->L.pool && i < kMaxPool; ++i) out->page_tokens[i] = tmp->page_tokens[i];
    free(tmp);
    return RPKV_OK;
}

int kv_get_info(const kv_handle* h, kv_info* out) {
    if (!h || !out) return RPKV_EINVAL;
    const Layout& L = h->L;
    out->num_layers = h->cfg.num_layers;
    out->num_streams = L.S;
    out->num_heads = L.H;
    out->head_dim = kHeadDim;
    out->dtype = h->cfg.dtype;
    out->tokens_per_frame = L.N;
    out->pool_pages = L.pool;
    out->slot_capacity = L.slot_cap;
    out->special_capacity = L.sp_cap;
    out->attn_splits = L.splits;
    out->page_bytes = (size_t)2 * L.H * L.slot_cap * kHeadDim * L.elem;
    out->cache_bytes = (size_t)2 * (L.kpool_elems + L.ksp_elems) * L.elem;
    out->total_bytes = L.total;
    out->off_kpool = L.off_kpool;
    out->off_vpool = L.off_vpool;
    out->off_ksp = L.off_ksp;
    out->off_vsp = L.off_vsp;
    out->frames_appended = h->appended;
    out->frames_committed = h->committed;
    return RPKV_OK;
}

const char* rpkv_strerror(int code) {
    switch (code) {
        case RPKV_OK: return "ok";
        case RPKV_EINVAL: return "invalid argument";
        case RPKV_EHIP: return "HIP runtime error";
        case RPKV_ENOSPACE: return "cache pool or special stream exhausted";
        case RPKV_ESTATE: return "invalid state";
        case RPKV_ETOOBIG: return "split scratch larger than the library's static scratch";
        default: return "unknown error";
    }
}

}  // extern "C"
