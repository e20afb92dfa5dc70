"""GPU parity of the fused projection + RoPE + append (kv_project_append_frame)
against the float64 oracle: the chain's projection (oracle.chain.project_qkv)
feeding the oracle stream's rotation, pages and attention.

Inputs: the chain's seeded hidden states N(0, 1) and projection weights
N(0, 0.02), both bf16; with these widths the projections stay below 2 in
magnitude, so a one-ulp difference in the stored projection (fp32 vs exact
accumulation landing on the other side of a bf16 rounding boundary) plus the
final rounding stays under the 2e-2 bar."""
import numpy as np
import pytest
import torch

import rope_paged_kv_amd as rp
from gpu_harness import make_cache, to_dev
from oracle import pages, rope3d
from oracle.chain import project_qkv
from oracle.stream import OracleStream
from rpkv_inputs import embeddings, projection, small_variants

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-2


def _views(cache, s):
    kp, vp, ks, vs = cache.pool_views()
    return kp[0, s], vp[0, s], ks[0, s], vs[0, s]


@pytest.mark.parametrize("name", ["small_proj", "small_proj_half"])
def test_project_append_matches_oracle(name):
    wl = small_variants()[name]
    S, H, D, C, N, P, ns = wl.streams, wl.heads, wl.head_dim, wl.hidden, wl.tokens, wl.patches, wl.n_special
    cache = make_cache(wl)
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    w = projection(wl, 0, n_out=3 * H * D)                    # [C, 3*H*D]
    w_dev = to_dev(w.T, torch.bfloat16)                       # linear-layer layout [3*H*D][C]
    proj = {}

    def source(s):
        def get(f, t):
            if (s, f) not in proj:
                proj[(s, f)] = project_qkv(embeddings(wl, s, f), w, H, D)
            return proj[(s, f)][t]
        return get

    orc = {s: OracleStream(wl, source(s)) for s in range(S)}
    shape = (S, N, H, D)
    q_rot = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, H, N), dtype=torch.float32, device="cuda")
    perm = np.array([rp.vslot_perm(p) for p in range(64)])
    for f in range(wl.frames):
        commit = wl.is_keyframe(f)
        x = np.stack([embeddings(wl, s, f) for s in range(S)])
        cache.project_append(0, f, int(commit), to_dev(x, torch.bfloat16), w_dev, q_rot)
        sim.append(f, commit)
        cache.attend(0, q_rot, out, lse)
        torch.cuda.synchronize()
        for s in range(S):
            st = cache.state(0, s)
            assert st["target_page"] == sim.target and st["special_offset"] == sim.sp_offset, (f, s)
            assert st["visible_pages"] == sim.visible.patch_pages, (f, s)
            assert st["visible_special_tokens"] == sim.visible.special_tokens, (f, s)
            assert st["query_tokens"] == N and st["page_tokens"][sim.target] == P, (f, s)
            want_q = orc[s].q_rot(f)
            assert np.abs(q_rot[s].float().cpu().numpy() - want_q).max() <= BF16_TOL, (f, s)
            want_k, want_v = orc[s].kv(f)
            kp, vp, ks, vs = _views(cache, s)
            t, o = sim.target, sim.sp_offset
            got_k = kp[:, t, :P].float().cpu().numpy().transpose(1, 0, 2)
            assert np.abs(got_k - want_k[ns:]).max() <= BF16_TOL, (f, s)
            got_ks = ks[:, o:o + ns].float().cpu().numpy().transpose(1, 0, 2)
            assert np.abs(got_ks - want_k[:ns]).max() <= BF16_TOL, (f, s)
            vt = vp[:, t].float().cpu().numpy()               # [H][D][cap]
            cap = vt.shape[-1]
            key_of_pos = (np.arange(cap) // 64) * 64 + perm[np.arange(cap) % 64]
            by_key = vt[:, :, np.argsort(key_of_pos)]
            assert np.abs(by_key[:, :, :P].transpose(2, 0, 1) - want_v[ns:]).max() <= BF16_TOL, (f, s)
            # the padding slots of the last written tile are zeros
            assert np.all(by_key[:, :, P:(P + 63) // 64 * 64] == 0), (f, s)
            spos = [(j // 64) * 64 + perm[j % 64] for j in range(o, o + ns)]
            got_vs = vs[:, :, spos].float().cpu().numpy().transpose(2, 0, 1)
            assert np.abs(got_vs - want_v[:ns]).max() <= BF16_TOL, (f, s)
            o_want, lse_want = orc[s].attend(f)
            assert np.abs(out[s].float().cpu().numpy() - o_want).max() <= BF16_TOL, (f, s)
            assert np.abs(lse[s].cpu().numpy() - lse_want).max() <= LSE_TOL, (f, s)
        sim.evict()
        cache.evict(0)


def test_project_append_checks_its_arguments():
    wl = small_variants()["small_proj"]
    cache = make_cache(wl)
    H, D, C, N = wl.heads, wl.head_dim, wl.hidden, wl.tokens
    x = torch.zeros((wl.streams, N, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3 * H * D, C), dtype=torch.bfloat16, device="cuda")
    q_rot = torch.empty((wl.streams, N, H, D), dtype=torch.bfloat16, device="cuda")
    for hidden in (0, 32, 96):
        with pytest.raises(rp.RpkvError):
            rp.kv_project_append_frame(cache.h, 0, 0, 1, x, hidden, w, q_rot, cache.tables, cache.stream)
    odd = make_cache(small_variants()["small_skip"])          # 3 heads
    with pytest.raises(rp.RpkvError):
        rp.kv_project_append_frame(odd.h, 0, 0, 1, x, C, w, q_rot, odd.tables, odd.stream)
    f32 = make_cache(small_variants()["small_f32"])
    with pytest.raises(rp.RpkvError):
        rp.kv_project_append_frame(f32.h, 0, 0, 1, x, C, w, q_rot, f32.tables, f32.stream)
    for grid in ((14, 17), (13, 18), (0, 5), (17, 13)):    # configured grid 13x17
        with pytest.raises(rp.RpkvError):
            cache.project_append(0, 0, 1, x, w, q_rot, grid=grid)


def test_project_append_shares_the_overflow_rule():
    """The fused path takes the same append target and frame record as
    kv_append_frame: a keyframe past max_keyframes sets the sticky
    ENOSPACE, later fused appends write nothing to the pages and show an empty
    visible set (attention: zeros, lse -inf), and a reset recovers."""
    wl = small_variants()["small_proj"]
    S, H, D, C, N = wl.streams, wl.heads, wl.head_dim, wl.hidden, wl.tokens
    cache = make_cache(wl, max_keyframes=2)
    x = torch.zeros((S, N, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3 * H * D, C), dtype=torch.bfloat16, device="cuda")
    q_rot = torch.empty((S, N, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q_rot)
    lse = torch.empty((S, H, N), dtype=torch.float32, device="cuda")
    for f in range(2):
        cache.project_append(0, f, 1, x, w, q_rot)
        cache.evict(0)
    assert all(cache.state(0, s)["status"] == 0 for s in range(S))
    cache.project_append(0, 2, 1, x, w, q_rot)
    cache.evict(0)                                        # a 3rd keyframe does not fit
    for s in range(S):
        st = cache.state(0, s)
        assert st["status"] == rp.RPKV_ENOSPACE and st["n_special_tokens"] == 12, s
    cache.project_append(0, 3, 1, x, w, q_rot)
    for s in range(S):
        st = cache.state(0, s)
        assert st["status"] == rp.RPKV_ENOSPACE and st["n_visible_pages"] == 0, s
    cache.attend(0, q_rot, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    cache.reset(0)
    cache.project_append(0, 0, 1, x, w, q_rot)
    for s in range(S):
        st = cache.state(0, s)
        assert st["status"] == 0 and st["target_page"] == 0 and st["visible_pages"] == [0], s


def test_project_append_variable_grids():
    """Frames of their own grids through the fused path (13x17, 11x17, 5x6,
    1x1, 13x9 in 13x17 pages): page token counts, q_rot of the frame's rows,
    K pages of the frame's patches and attention of its tokens against the
    oracle; rows past the frame keep what they held."""
    wl = small_variants()["small_proj"].replace(grids=((13, 17), (11, 17), (5, 6), (1, 1), (13, 9)),
                                                frames=7)
    S, H, D, ns = wl.streams, wl.heads, wl.head_dim, wl.n_special
    cache = make_cache(wl)
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    w = projection(wl, 0, n_out=3 * H * D)
    w_dev = to_dev(w.T, torch.bfloat16)
    proj = {}

    def source(s):
        def get(f, t):
            if (s, f) not in proj:
                proj[(s, f)] = project_qkv(embeddings(wl, s, f), w, H, D)
            return proj[(s, f)][t]
        return get

    orc = {s: OracleStream(wl, source(s)) for s in range(S)}
    shape = (S, wl.tokens, H, D)
    q_rot = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, H, wl.tokens), dtype=torch.float32, device="cuda")
    for f in range(wl.frames):
        gh, gw = wl.grid_of(f)
        n, commit = ns + gh * gw, wl.is_keyframe(f)
        x = np.stack([embeddings(wl, s, f) for s in range(S)])
        q_rot.fill_(7.0)
        out.fill_(7.0)
        cache.project_append(0, f, int(commit), to_dev(x, torch.bfloat16), w_dev, q_rot, grid=(gh, gw))
        sim.append(f, commit)
        cache.attend(0, q_rot, out, lse)
        torch.cuda.synchronize()
        want_pt = {p: wl.grid_of(g)[0] * wl.grid_of(g)[1] for p, g in sim.page_frame.items()}
        want_pt[sim.target] = gh * gw
        for s in range(S):
            st = cache.state(0, s)
            assert st["query_tokens"] == n and st["visible_pages"] == sim.visible.patch_pages, (f, s)
            for p, cnt in want_pt.items():
                assert st["page_tokens"][p] == cnt, (f, s, p)
            assert np.abs(q_rot[s, :n].float().cpu().numpy() - orc[s].q_rot(f)).max() <= BF16_TOL, (f, s)
            assert torch.all(q_rot[s, n:] == 7.0) and torch.all(out[s, n:] == 7.0), (f, s)
            kp = _views(cache, s)[0]
            got_k = kp[:, sim.target, :gh * gw].float().cpu().numpy().transpose(1, 0, 2)
            assert np.abs(got_k - orc[s].kv(f)[0][ns:]).max() <= BF16_TOL, (f, s)
            o_want, lse_want = orc[s].attend(f)
            assert np.abs(out[s, :n].float().cpu().numpy() - o_want).max() <= BF16_TOL, (f, s)
            assert np.abs(lse[s, :, :n].cpu().numpy() - lse_want).max() <= LSE_TOL, (f, s)
        sim.evict()
        cache.evict(0)


@pytest.mark.parametrize("n", [5, 8 * 37 + 3, 4 * 1375 * 1024])
def test_residual_add_is_the_fp32_sum_and_its_bf16_rounding(n):
    """residual_add_bf16 against its definition on the CPU: x + o in fp32,
    then round to nearest even into bf16 -- bit for bit, at a length below
    one 8-element chunk, one with a ragged tail, and the full-depth
    workload's [4][1375][1024].  Values span bf16 rounding ties and sums that
    overflow to inf."""
    g = torch.Generator().manual_seed(n)
    x = torch.randn(n, generator=g) * 3
    o = (torch.randn(n, generator=g) * 3).to(torch.bfloat16)
    x[:2] = torch.tensor([3.0e38, 1.0 + 2.0 ** -8])         # overflow; a tie of bf16 rounding
    o[:2] = torch.tensor([3.0e38, 0.0]).to(torch.bfloat16)
    want_x = x + o.float()
    want_xb = want_x.to(torch.bfloat16)
    xd, od = x.cuda(), o.cuda()
    xbd = torch.full((n,), 7.0, dtype=torch.bfloat16, device="cuda")
    rp.residual_add(xd, od, xbd)
    torch.cuda.synchronize()
    assert torch.equal(xd.cpu().view(torch.int32), want_x.view(torch.int32))
    assert torch.equal(xbd.cpu().view(torch.int16), want_xb.view(torch.int16))
    # without the cast: x only, nothing else written
    xd2 = x.cuda()
    rp.residual_add(xd2, od, None)
    torch.cuda.synchronize()
    assert torch.equal(xd2.cpu().view(torch.int32), want_x.view(torch.int32))
