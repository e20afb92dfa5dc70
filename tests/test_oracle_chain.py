"""Pin of the full-depth chain oracle (frame-major, with per-layer caches)
against an independent layer-major formulation: all frames of a layer at once,
attention as PyTorch SDPA on the CPU under an explicit visibility mask, heads
split by the usual [N, 3, H, D] view of the projection output."""
import numpy as np
import torch

from oracle import retained, rope3d
from oracle.chain import OracleChain
from rpkv_inputs import embeddings, projection, small_variants


def layer_major(wl, stream):
    n, h, d, hid = wl.tokens, wl.heads, wl.head_dim, wl.hidden
    fr = wl.frames
    x = torch.from_numpy(np.concatenate([embeddings(wl, stream, f) for f in range(fr)]).astype(np.float64))
    owner = np.repeat(np.arange(fr), n)
    tok = np.tile(np.arange(n), fr)
    # visibility of key (g, t) to query frame f on a cached layer
    allow = np.zeros((fr * n, fr * n), dtype=bool)
    for f in range(fr):
        pf, spf = retained.visible_for_schedule(f, wl.keyframe_interval, wl.scale_frames,
                                                wl.sliding_window)
        kmask = (np.isin(owner, pf) & (tok >= wl.n_special)) | (np.isin(owner, spf) & (tok < wl.n_special))
        allow[owner == f] = kmask
    frame_mask = owner[:, None] == owner[None, :]
    tabs = [rope3d.rotation_table(rope3d.token_positions(f, wl.grid_h, wl.grid_w, wl.n_special),
                                  wl.pairs, wl.theta) for f in range(fr)]
    outs = []
    for layer in range(wl.chain_layers):
        w = torch.from_numpy(projection(wl, layer).astype(np.float64))
        qkv = (x @ w).view(fr * n, 3, h, d).numpy()
        q = np.concatenate([rope3d.apply_rotary(qkv[owner == f, 0], tabs[f]) for f in range(fr)])
        k = np.concatenate([rope3d.apply_rotary(qkv[owner == f, 1], tabs[f]) for f in range(fr)])
        v = qkv[:, 2]
        mask = frame_mask if layer % 2 == 0 else allow
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
            torch.from_numpy(np.ascontiguousarray(v)).transpose(0, 1),
            attn_mask=torch.from_numpy(mask)).transpose(0, 1)
        outs.append(o.numpy())
        x = x + o.reshape(fr * n, hid)
    return outs, x.numpy(), owner


def test_chain_matches_layer_major_formulation():
    wl = small_variants()["small_chain"].replace(dtype="f32")
    for stream in (0, 1):
        outs, xl, owner = layer_major(wl, stream)
        ch = OracleChain(wl, lambda f: embeddings(wl, stream, f), lambda l: projection(wl, l))
        for f in range(wl.frames):
            o_f, x_f = ch.frame(f)
            for layer in range(wl.chain_layers):
                np.testing.assert_allclose(o_f[layer], outs[layer][owner == f], atol=1e-12)
            np.testing.assert_allclose(x_f, xl[owner == f], atol=1e-11)


def test_bf16_chain_close_to_f32_chain():
    # the bf16 storage rounding only perturbs the chain slightly
    wl = small_variants()["small_chain"]
    a = OracleChain(wl, lambda f: embeddings(wl, 0, f), lambda l: projection(wl, l))
    b = OracleChain(wl.replace(dtype="f32"), lambda f: embeddings(wl, 0, f), lambda l: projection(wl, l))
    for f in range(3):
        _, xa = a.frame(f)
        _, xb = b.frame(f)
        assert np.abs(xa - xb).max() < 2e-2


def test_project_qkv_on_one_hot_rows_returns_the_weight_rows():
    """Token i = e_i picks row i of W: Q, K, V of token i are the three thirds
    of that row, head h at columns h*D .. h*D+D-1 of each third, rounded once
    to bf16 (the weights are bf16 already, so exactly the row)."""
    from oracle.chain import project_qkv
    rng = np.random.default_rng(7)
    H, D, C = 2, 4, 8
    w = rope3d.round_bf16(rng.standard_normal((C, 3 * H * D)))
    q, k, v = project_qkv(np.eye(C), w, H, D)
    for i in range(C):
        for t, got in enumerate((q, k, v)):
            for h in range(H):
                np.testing.assert_array_equal(got[i, h], w[i, t * H * D + h * D:t * H * D + (h + 1) * D])
    # two one-hot tokens: their sum (exact in float64) rounded once to bf16
    q2, k2, v2 = project_qkv(np.eye(C)[0] + np.eye(C)[[1]], w, H, D)
    for t, got in enumerate((q2, k2, v2)):
        want = rope3d.round_bf16(w[0, t * H * D:(t + 1) * H * D] + w[1, t * H * D:(t + 1) * H * D])
        np.testing.assert_array_equal(got[0].reshape(H * D), want)
        assert np.any(want != w[0, t * H * D:(t + 1) * H * D] + w[1, t * H * D:(t + 1) * H * D])
