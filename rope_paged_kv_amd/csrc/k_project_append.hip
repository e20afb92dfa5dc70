// Fused QKV projection + 3D rotary embedding + paged KV append, bf16.
//
// What is computed.  The rotary embedding is applied to Q and K right after
// their projection and before the cache write (page "How 3D RoPE Positional
// Encoding Works with the Paged KV Cache in LingBot-Map", FAQ on where the RoPE
// application sits relative to the KV cache write).  For every stream s:
//  * [Q | K | V] = X_s W^T, X_s the frame's hidden states [N][C] and W the
//    layer's projection [3*H*D][C] as a linear layer stores it (no bias); each
//    product is accumulated in fp32 and rounded once to bf16 -- the bf16
//    projection output the cache path starts from;
//  * then exactly what kv_append_frame does with that Q, K, V: Q and K rotated
//    at their tokens' (t, h, w) positions (fp32, rounded once), rotated Q to
//    q_rot, rotated K and raw V of the patches to the frame's patch page and of
//    the 6 specials to the special stream, the same target, frame record and
//    pending commit (shared code: rope_rows.h).
// The round trip of Q, K and V through HBM between a projection GEMM and the
// append kernel is gone: the products go from the matrix cores through LDS
// straight to q_rot and the pages.
//
// Layout of the work:
//  * a workgroup of 4 waves computes a 128 x 128 tile of the transposed
//    product (W X^T): 128 output channels -- two heads of one of Q, K, V --
//    by 128 token rows; each wave one head by 64 rows, as 2 x 2 blocks of
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 64 registers);
//  * token rows are taken in "virtual" order: the frame's patches first, then
//    its 6 specials, so the specials fill the spare rows of the last patch
//    tile instead of costing a tile of their own, and every wave's 64 patch
//    rows are exactly one 64-slot tile of the page;
//  * the reduction walks C in steps of 64 through two LDS stages (32 KB each:
//    the W and X tiles, 16-byte chunks XOR-swizzled by row so the operand
//    reads of 32 rows hit distinct banks); the next step's global loads are in
//    flight while the current one is multiplied, one barrier per step;
//  * epilogue per wave: the bf16 products go to LDS, token-major for Q and K
//    (then every lane rotates whole 16-byte chunks -- both chunks of a pair in
//    the half-split layout -- and stores them with full-width writes) or
//    transposed at their storage positions for V (the page's V^T rows are then
//    written 128 bytes at a time; slots past the frame's patches are zeros);
//  * the first workgroup of each stream writes the frame record.
#include "rope_rows.h"

namespace rpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPM = 128;                       // token rows per workgroup
constexpr int kPN = 128;                       // output channels per workgroup (two heads)
constexpr int kPK = 64;                        // reduction depth per LDS stage
constexpr int kOpBytes = 128 * kPK * 2;        // one operand tile of a stage: 16 KB
constexpr int kStageBytes = 2 * kOpBytes;      // W tile then X tile
constexpr int kPitch = kHeadDim + 8;           // staging row pitch in elements (144 B)

// Byte offset of 16-byte chunk c (of 8) of row r in an operand tile.  A
// 128-byte row covers half of the 64 LDS banks, so 16 consecutive rows (the
// lanes an operand read serves together) reach every bank group once when
// chunk c of row r sits at position c ^ ((r >> 1) & 7).
__device__ inline int op_off(int r, int c) { return r * (kPK * 2) + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ inline uint16_t bf16_rne(float x) {   // finite input
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int LAYOUT>
__global__ __launch_bounds__(256, 2) void k_project_append(ProjArgs p) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];
    const AppendArgs& a = p.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wo = wave & 1, wv = wave >> 1;   // head of the pair, 64-row half
    const int cb = blockIdx.x % p.col_blocks, rb = blockIdx.x / p.col_blocks, s = blockIdx.y;
    const int nvalid = a.fP + a.nsp;           // virtual rows: patches, then specials

    // Global -> LDS: thread tid moves chunk (tid & 7) of rows (tid >> 3) + 32 i
    // of both operand tiles; rows past the frame's tokens read token 0.
    const int lr = tid >> 3, lc = tid & 7;
    const uint16_t* xs0 = p.x;
    const uint16_t* ws0 = p.w + (size_t)(cb * kPN + lr) * p.C + lc * 8;
    const size_t wstep = (size_t)32 * p.C;   // W rows lr + 32 i
    size_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int v = rb * kPM + lr + 32 * i;
        const int tok = v < a.fP ? a.nsp + v : (v < nvalid ? v - a.fP : 0);
        xoff[i] = ((size_t)s * a.N + tok) * p.C + lc * 8;
    }
    // (named registers: an array of these ends up in scratch memory)
    uint4 rw0, rw1, rw2, rw3, rx0, rx1, rx2, rx3;
#define PROJ_GLOAD(k0)                                                   \
    {                                                                    \
        rw0 = *(const uint4*)(ws0 + (k0));                               \
        rw1 = *(const uint4*)(ws0 + wstep + (k0));                       \
        rw2 = *(const uint4*)(ws0 + 2 * wstep + (k0));                   \
        rw3 = *(const uint4*)(ws0 + 3 * wstep + (k0));                   \
        rx0 = *(const uint4*)(xs0 + xoff[0] + (k0));                     \
        rx1 = *(const uint4*)(xs0 + xoff[1] + (k0));                     \
        rx2 = *(const uint4*)(xs0 + xoff[2] + (k0));                     \
        rx3 = *(const uint4*)(xs0 + xoff[3] + (k0));                     \
    }
#define PROJ_LSTORE(buf)                                                 \
    {                                                                    \
        char* A_ = lds + (buf) * kStageBytes;                            \
        *(uint4*)(A_ + op_off(lr, lc)) = rw0;                            \
        *(uint4*)(A_ + op_off(lr + 32, lc)) = rw1;                       \
        *(uint4*)(A_ + op_off(lr + 64, lc)) = rw2;                       \
        *(uint4*)(A_ + op_off(lr + 96, lc)) = rw3;                       \
        *(uint4*)(A_ + kOpBytes + op_off(lr, lc)) = rx0;                 \
        *(uint4*)(A_ + kOpBytes + op_off(lr + 32, lc)) = rx1;            \
        *(uint4*)(A_ + kOpBytes + op_off(lr + 64, lc)) = rx2;            \
        *(uint4*)(A_ + kOpBytes + op_off(lr + 96, lc)) = rx3;            \
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = p.C / kPK;
    const int arow = 64 * wo + (lane & 31), brow = 64 * wv + (lane & 31), khalf = lane >> 5;
    PROJ_GLOAD(0)
    PROJ_LSTORE(0)
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) {
            PROJ_GLOAD((kt + 1) * kPK)
        }
        const char* A = lds + (kt & 1) * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < kPK / 16; ++ks) {
            bf16x8 af[2], bf[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                af[j] = *(const bf16x8*)(A + op_off(arow + 32 * j, 2 * ks + khalf));
                bf[j] = *(const bf16x8*)(A + kOpBytes + op_off(brow + 32 * j, 2 * ks + khalf));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            PROJ_LSTORE((kt + 1) & 1)
        }
        __syncthreads();
    }
#undef PROJ_GLOAD
#undef PROJ_LSTORE

    // Epilogue.  acc[i][j] register e holds channel 32 i + 8 (e / 4) +
    // 4 (lane / 32) + e % 4 of this wave's head, token row 32 j + lane % 32 of
    // this wave's 64 rows (virtual rows V0 ..).
    const int HD = a.H * kHeadDim;
    const int part = (cb * kPN) / HD;                            // 0 Q, 1 K, 2 V
    const int head = (cb * kPN - part * HD) / kHeadDim + wo;
    const int V0 = rb * kPM + 64 * wv;
    CacheState* st = a.states + s;
    const Target tg = append_target(a, st);
    uint16_t* stg = (uint16_t*)lds + wave * (64 * kPitch);      // this wave's 64 x 72 staging tile

    // Q and K: this lane rotates NSLOT chunk slots (interleaved: chunk lane % 8
    // of rows lane / 8 + 8 i; half-split: pair slot lane % 4 of rows lane / 4
    // + 16 i).  Their rotation coefficients are loaded first, so that the
    // loads are in flight while the products are staged.
    constexpr bool kInter = LAYOUT == RPKV_ROPE_INTERLEAVED;
    constexpr int NSLOT = kInter ? 8 : 4, NCO = kInter ? 4 : 8;
    float2 cw[NSLOT][NCO];
    if (part < 2) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int row = kInter ? (lane >> 3) + 8 * i : (lane >> 2) + 16 * i;
            const int c = kInter ? (lane & 7) : pair_chunk<8>(a, lane & 3, 0);
            const int V = V0 + row;
            int hp = 0, wp = 0;   // specials (and rows past the frame) sit at h = w = 0
            if (V < a.fP) {
                hp = V / a.fgw;
                wp = V - hp * a.fgw;
            }
#pragma unroll
            for (int e = 0; e < NCO; ++e) cw[i][e] = coeff_of<8, LAYOUT>(a, c, e, hp, wp);
        }
    }

    if (part < 2) {
        // token-major: stg[row][channel]
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int o = 32 * i + 8 * g + 4 * khalf, v = 32 * j + (lane & 31);
                    const uint32_t lo = bf16_rne(acc[i][j][4 * g]) | ((uint32_t)bf16_rne(acc[i][j][4 * g + 1]) << 16);
                    const uint32_t hi = bf16_rne(acc[i][j][4 * g + 2]) | ((uint32_t)bf16_rne(acc[i][j][4 * g + 3]) << 16);
                    *(uint2*)(stg + v * kPitch + o) = make_uint2(lo, hi);
                }
    } else {
        // V: stg[channel][storage position of the row's slot]; rows that are
        // not patches of this frame leave zeros (padding slots), specials go
        // to the special stream from here.
        uint16_t* vsp = (uint16_t*)a.vsp + s * a.ksp_elems + (size_t)head * kHeadDim * a.sp_cap;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int v = 32 * j + (lane & 31), V = V0 + v;
                const bool patch = V < a.fP;
                const bool special = !patch && V < nvalid && tg.ok;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int o = 32 * i + 8 * (e >> 2) + 4 * khalf + (e & 3);
                    const uint16_t b = bf16_rne(acc[i][j][e]);
                    stg[o * kPitch + vslot_perm(v)] = patch ? b : (uint16_t)0;
                    if (special) vsp[(size_t)o * a.sp_cap + vslot_perm(tg.sp_off + V - a.fP)] = b;
                }
            }
    }
    __syncthreads();

    if (part < 2) {
        const size_t rs = (size_t)a.H * kHeadDim;
        uint16_t* qdst = (uint16_t*)a.q_rot + (size_t)s * a.N * rs + (size_t)head * kHeadDim;
        uint16_t* kpage = (uint16_t*)a.kpool + s * a.kpool_elems +
                          ((size_t)head * a.pool + tg.page) * a.slot_cap * kHeadDim;
        uint16_t* kspb = (uint16_t*)a.ksp + s * a.ksp_elems + ((size_t)head * a.sp_cap + tg.sp_off) * kHeadDim;
        // q_rot is read by the attention right after; K rows stream to the page.
        auto put = [&](uint16_t* dst, const uint4& v) {
            if (part == 0)
                *(uint4*)dst = v;
            else
                store_stream(dst, v);
        };
        // Destination of row `row` of this wave (null: nothing to write).
        auto dst_row = [&](int row) -> uint16_t* {
            const int V = V0 + row;
            if (V >= nvalid) return nullptr;
            const bool patch = V < a.fP;
            if (part == 0) return qdst + (size_t)(patch ? a.nsp + V : V - a.fP) * rs;
            if (!tg.ok) return nullptr;
            return patch ? kpage + (size_t)V * kHeadDim : kspb + (size_t)(V - a.fP) * kHeadDim;
        };
        if (kInter) {
#pragma unroll
            for (int i = 0; i < NSLOT; ++i) {
                const int row = (lane >> 3) + 8 * i, c = lane & 7;
                uint16_t* d = dst_row(row);
                if (!d) continue;
                float f[8];
                Vec<uint16_t>::unpack(*(const uint4*)(stg + row * kPitch + c * 8), f);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float2 w = cw[i][e];
                    const float x = f[2 * e], y = f[2 * e + 1];
                    f[2 * e] = x * w.x - y * w.y;
                    f[2 * e + 1] = x * w.y + y * w.x;
                }
                put(d + c * 8, Vec<uint16_t>::pack(f));
            }
        } else {
            const int c0 = pair_chunk<8>(a, lane & 3, 0), c1 = pair_chunk<8>(a, lane & 3, 1);
#pragma unroll
            for (int i = 0; i < NSLOT; ++i) {
                const int row = (lane >> 2) + 16 * i;
                uint16_t* d = dst_row(row);
                if (!d) continue;
                float f0[8], f1[8];
                Vec<uint16_t>::unpack(*(const uint4*)(stg + row * kPitch + c0 * 8), f0);
                Vec<uint16_t>::unpack(*(const uint4*)(stg + row * kPitch + c1 * 8), f1);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float2 w = cw[i][e];
                    const float x = f0[e], y = f1[e];
                    f0[e] = x * w.x - y * w.y;
                    f1[e] = y * w.x + x * w.y;
                }
                put(d + c0 * 8, Vec<uint16_t>::pack(f0));
                put(d + c1 * 8, Vec<uint16_t>::pack(f1));
            }
        }
    } else if (V0 < a.fP && tg.ok) {
        // V^T rows of the page: channel d, storage positions V0 .. V0+63.
        uint16_t* vpage = (uint16_t*)a.vpool + s * a.kpool_elems +
                          ((size_t)head * a.pool + tg.page) * kHeadDim * a.slot_cap + V0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = lane + 64 * i, d = id >> 3, g = id & 7;
            store_stream(vpage + (size_t)d * a.slot_cap + g * 8, *(const uint4*)(stg + d * kPitch + g * 8));
        }
    }

    if (blockIdx.x == 0) write_frame_record(a, st, tg, tid);
}

hipError_t launch_project_append(const ProjArgs& p, hipStream_t st) {
    dim3 grid(p.col_blocks * p.row_blocks, p.a.S);
    if (p.a.layout == RPKV_ROPE_HALF_SPLIT)
        hipLaunchKernelGGL(k_project_append<RPKV_ROPE_HALF_SPLIT>, grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL(k_project_append<RPKV_ROPE_INTERLEAVED>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace rpkv
