"""Pins for the oracle's sparse attention and layer-group schedule (CPU only):
closed forms, a library attention routine on the same gathered rows, causal
poison, Reuse byte identity and the layer layout the pages print."""

import json
import os

import numpy as np
import torch

from oracle import attention as A
from oracle import formats as Fm
from oracle import group as G
from oracle import indexer as I

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_cache(rng, n):
    y = rng.standard_normal((n, 512)).astype(np.float32)
    return Fm.quantize_rows(y)


def _rand_swa(rng, s):
    x = torch.from_numpy(rng.standard_normal((s, 512)).astype(np.float32))
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_zero_query_gives_mean_of_keys():
    rng = np.random.default_rng(0)
    cache = _rand_cache(rng, 64)
    swa = _rand_swa(rng, 200)
    idx = np.full(512, -1, dtype=np.int32)
    idx[:40] = np.sort(rng.choice(64, 40, replace=False))
    out = A.sparse_attention(np.zeros((64, 512)), cache, idx, swa, t=150, swa_pos0=0)
    keys = np.concatenate([Fm.dequantize_rows(cache[idx[:40]]),
                           Fm.e4m3_decode(swa[23:151])])
    assert keys.shape[0] == 40 + 128
    want = keys.mean(axis=0).astype(np.float32)
    assert np.allclose(out, want[None, :], rtol=0, atol=1e-6)


def test_single_key_returns_that_row():
    rng = np.random.default_rng(1)
    swa = _rand_swa(rng, 4)
    idx = np.full(512, -1, dtype=np.int32)
    q = rng.standard_normal((64, 512))
    out = A.sparse_attention(q, _rand_cache(rng, 8), idx, swa, t=0, swa_pos0=0)
    assert np.array_equal(out, np.broadcast_to(Fm.e4m3_decode(swa[0]).astype(np.float32), (64, 512)))


def test_matches_torch_sdpa_on_gathered_rows():
    rng = np.random.default_rng(2)
    cache = _rand_cache(rng, 1000)
    swa = _rand_swa(rng, 300)
    idx = np.sort(rng.choice(1000, 512, replace=False)).astype(np.int32)
    q = rng.standard_normal((64, 512)) / np.sqrt(512)
    t, pos0 = 1200, 1000
    out = A.sparse_attention(q, cache, idx, swa, t=t, swa_pos0=pos0, scale=0.7)
    keys = torch.from_numpy(A.gather_keys(cache, idx, swa, t, pos0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], keys[None], keys[None], scale=0.7)[0]
    assert np.allclose(out, ref.numpy(), rtol=1e-6, atol=1e-6)


def test_split_merge_by_log_sum_exp_equals_unsplit():
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((640, 512))
    q = rng.standard_normal((64, 512)) / 20
    full = A.softmax_attention(q, keys, 1.0)
    parts = []
    for a in range(0, 640, 96):
        z = q @ keys[a:a + 96].T
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        parts.append((m, p.sum(axis=1, keepdims=True), p @ keys[a:a + 96]))
    M = np.max([m for m, _, _ in parts], axis=0)
    L = sum(l * np.exp(m - M) for m, l, _ in parts)
    O = sum(o * np.exp(m - M) for m, _, o in parts) / L
    assert np.allclose(full, O, rtol=1e-12, atol=1e-12)


def test_window_bounds():
    assert A.swa_tokens(0).tolist() == [0]
    assert A.swa_tokens(5).tolist() == list(range(6))
    w = A.swa_tokens(1048575)
    assert w[0] == 1048575 - 127 and w[-1] == 1048575 and len(w) == 128


# ------------------------------------------------------------------ group -----

def test_layout_matches_pages():
    with open(os.path.join(GOLD, "pages_facts.json")) as f:
        facts = json.load(f)
    lay = G.model_layout()
    modes = {L: v[0] for L, v in lay.items() if v is not None}
    full_layers = sorted(L for L, m in modes.items() if m == G.FULL)
    # the pages' four KV-generating layers, read as 0-based numbers
    assert [L - 1 for L in full_layers] == facts["layout"]["kv_generating_layers_as_printed"]
    enc = [modes[L] for L in range(3, 21)]
    assert enc == facts["layout"]["encoder"]["group"] * 3
    dec = [modes[L] for L in range(21, 41)]
    assert dec == facts["layout"]["decoder"]["first_group"] + facts["layout"]["decoder"]["other_groups"] * 4
    assert all(lay[L][1] == 2 for L in range(3, 21)) and all(lay[L][1] == 1 for L in range(21, 41))
    # KV entries per token: three m=2 Full layers and one m=1 Full layer
    assert sum(1.0 / lay[L][1] for L in full_layers) == 2.5
    assert Fm.ROW_BYTES == 288
    # the printed 890 B/token leaves 890/2.5 - 288 = 68 B per entry for the
    # indexer key, which is a 128-wide FP4 key (64 B) plus 4 scale bytes
    assert facts["bytes_per_token"]["global_kv"] / 2.5 - Fm.ROW_BYTES == 64 + 4


def test_mode_table_semantics_in_schedule():
    with open(os.path.join(GOLD, "pages_facts.json")) as f:
        table = json.load(f)["mode_table"]
    sched = G.layer_schedule("decoder")
    assert [m for m, _ in sched] == ["F", "X", "U", "X", "U", "X", "U"]
    for li, (m, src) in enumerate(sched):
        row = table[m]
        assert (src is None) == (row[0] == "own")           # main KV
        if m == "U":
            assert sched[src][0] in ("F", "X")              # reuses indices
    assert [m for m, _ in G.layer_schedule("encoder")] == ["F"] + ["U"] * 5


def _group_inputs(rng, n_cap, n_layers, S):
    k = _rand_swa(rng, n_cap)[:, :128].copy()
    cache = _rand_cache(rng, n_cap)
    qi = {l: _rand_swa(rng, 32)[:, :128].copy() for l in range(n_layers)}
    w = {l: (rng.uniform(0, 1, 32) / 32).astype(np.float32) for l in range(n_layers)}
    q = {l: rng.standard_normal((64, 512)) / np.sqrt(512) for l in range(n_layers)}
    swa = {l: _rand_swa(rng, S) for l in range(n_layers)}
    return k, cache, qi, w, q, swa


def test_reuse_is_byte_identical_and_sources_untouched():
    sched = G.layer_schedule("decoder")
    idx, out, pool, _ = _run(_decoder_case(5))
    snap = {l: idx[l].copy() for l in idx}
    for li, (m, src) in enumerate(sched):
        if m == "U":
            assert idx[li].tobytes() == idx[src].tobytes()
    assert all(np.array_equal(snap[l], idx[l]) for l in idx)
    assert (pool >= 0).sum() == 2048
    for li in (1, 3, 5):
        assert all(int(p) // 8 in set(pool.tolist()) for p in idx[li])


def test_causal_poison_never_selected_and_never_changes_outputs():
    rng = np.random.default_rng(6)
    n_cap, n_vis = 6000, 4500
    k, cache, qi, w, q, swa = _group_inputs(rng, n_cap, 7, 256)
    t = n_vis - 1
    base = G.run_group(G.layer_schedule("decoder"), qi, w, q, swa, k, cache,
                       n_vis=n_vis, t=t, swa_pos0=t - 127)
    k2 = k.copy()
    k2[n_vis:] = 0x7E                     # +448 everywhere beyond n_vis
    c2 = cache.copy()
    c2[n_vis:, 256:] = 0x7F               # NaN scales beyond n_vis
    s2 = {l: v.copy() for l, v in swa.items()}
    for l in s2:
        s2[l][128:] = 0x7F                # NaN window rows after token t
    pois = G.run_group(G.layer_schedule("decoder"), qi, w, q, s2, k2, c2,
                       n_vis=n_vis, t=t, swa_pos0=t - 127)
    for l in base[0]:
        assert np.array_equal(base[0][l], pois[0][l])
        assert np.all(base[0][l] < n_vis)
        assert np.array_equal(base[1][l], pois[1][l])
    assert np.array_equal(base[2], pois[2])


def test_full_scores_block_max_consistent():
    rng = np.random.default_rng(7)
    k, cache, qi, w, q, swa = _group_inputs(rng, 300, 1, 128)
    s = I.index_scores(qi[0], w[0], k, n_vis=250)
    bm = I.block_max(s, 250)
    assert bm.shape[0] == 38
    for b in range(38):
        vis = s[8 * b:min(8 * b + 8, 250)]
        assert bm[b] == (vis.max() if vis.size else -np.inf)


# ------------------------------------------------- per-layer routing pins -----
# The pages fix that a Reindex layer scores with its own indexer query and that
# every layer computes its own main query and window KV ("DeepSeek V4.1-Flash
# 为什么这么强？", §二 mode table; "DeepSeek V4.1 Flash vs V4 Pro", 黑科技之二).

def _decoder_case(seed, n_cap=20000):
    # 20,000 positions = 2,500 blocks, so the 2,048-block pool is a strict subset
    rng = np.random.default_rng(seed)
    k = _rand_swa(rng, n_cap)[:, :128].copy()
    # packed rows drawn directly: any E2M1 code byte, E4M3 scales 2^-3 .. 1.875
    cache = np.concatenate([rng.integers(0, 256, (n_cap, 256)),
                            rng.integers(0x20, 0x40, (n_cap, 32))], axis=1).astype(np.uint8)
    qi = {l: _rand_swa(rng, 32)[:, :128].copy() for l in range(7)}
    w = {l: (rng.uniform(0, 1, 32) / 32).astype(np.float32) for l in range(7)}
    q = {l: rng.standard_normal((64, 512)) / np.sqrt(512) for l in range(7)}
    swa = {l: _rand_swa(rng, 128) for l in range(7)}
    t = n_cap - 1
    return dict(k=k, cache=cache, qi=qi, w=w, q=q, swa=swa, n_vis=n_cap, t=t, pos0=t - 127)


def _run(c, **over):
    a = dict(c)
    a.update(over)
    return G.run_group(G.layer_schedule("decoder"), a["qi"], a["w"], a["q"], a["swa"], a["k"],
                       a["cache"], n_vis=a["n_vis"], t=a["t"], swa_pos0=a["pos0"])


def test_reindex_with_the_full_layers_query_reproduces_its_topk():
    # the Full Top-512 lies inside the pool, so a Reindex layer given the Full
    # layer's indexer query must pick exactly the Full layer's set
    c = _decoder_case(20)
    qi = {l: c["qi"][0] for l in c["qi"]}
    w = {l: c["w"][0] for l in c["w"]}
    idx, _, pool, _ = _run(c, qi=qi, w=w)
    assert (pool >= 0).sum() == 2048 < -(-c["n_vis"] // 8)
    for li in (1, 3, 5):
        assert np.array_equal(idx[li], idx[0])


def test_each_reindex_layer_scores_with_its_own_indexer_query():
    c = _decoder_case(21)
    idx = _run(c)[0]
    sets = [frozenset(idx[li].tolist()) for li in (0, 1, 3, 5)]
    assert len(set(sets)) == 4
    # exchanging two Reindex layers' indexer queries exchanges their selections
    # (and their Reuse layers'), leaving the others alone
    qi, w = dict(c["qi"]), dict(c["w"])
    qi[1], qi[3] = c["qi"][3], c["qi"][1]
    w[1], w[3] = c["w"][3], c["w"][1]
    sw = _run(c, qi=qi, w=w)[0]
    for a, b in ((0, 0), (1, 3), (2, 4), (3, 1), (4, 2), (5, 5), (6, 6)):
        assert np.array_equal(sw[a], idx[b]), (a, b)


def test_each_layer_attends_with_its_own_query():
    # a zero query gives the plain mean of the layer's own keys (closed form);
    # only the one layer given a real query may differ from it
    c = _decoder_case(22)
    zero = np.zeros((64, 512))
    for R in (0, 3, 6):
        q = {l: zero for l in range(7)}
        q[R] = c["q"][R]
        idx, out, _, _ = _run(c, q=q)
        for li in range(7):
            mean = A.gather_keys(c["cache"], idx[li], c["swa"][li], c["t"], c["pos0"]).mean(axis=0)
            close = np.allclose(out[li], mean[None, :], rtol=0, atol=1e-6)
            assert close == (li != R), (R, li)


def test_each_layer_attends_over_its_own_window():
    # main rows all zero and a constant window row a_l per layer: every head's
    # logits are 0 for the 512 selected rows and a_l * sum_c q_hc for the 128
    # window rows, so out[h] = a_l * 128 e^{a_l s_h} / (512 + 128 e^{a_l s_h})
    c = _decoder_case(23)
    cache = np.zeros_like(c["cache"])
    vals = [0.5, 1.0, 1.5, 2.0, 3.0, -1.0, -2.5]
    codes = torch.tensor(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    swa = {l: np.full((128, 512), codes[l], dtype=np.uint8) for l in range(7)}
    _, out, _, _ = _run(c, cache=cache, swa=swa)
    for li in range(7):
        a = vals[li]
        s = c["q"][li].sum(axis=1)
        e = 128.0 * np.exp(a * s)
        want = (a * e / (512.0 + e))[:, None] * np.ones((1, 512))
        assert np.allclose(out[li], want, rtol=1e-6, atol=1e-7), li


# --------------------------------- window buffer: skip rules and ring layout ---

def test_out_of_range_indices_and_unheld_window_tokens_are_skipped():
    # constant rows: selected main rows hold 3.0 (scale 0.5, code 6: exact),
    # window rows 2.0; a zero query
    # averages exactly the keys that count, so the output names their number.
    # 7 indices lie in [0, 64); 5 do not. The query at t = 300 has window
    # tokens 173..300, of which the 40-row buffer from token 250 holds 250..289.
    one = Fm.quantize_rows(np.full((64, 512), 3.0, dtype=np.float32))
    assert np.all(Fm.dequantize_rows(one) == 3.0)
    idx = np.full(512, -1, dtype=np.int32)
    idx[:12] = [0, 3, 5, 9, 20, 33, 63, 64, 100, -7, 2**31 - 1, -(2**31)]
    two = np.full((40, 512), torch.tensor([2.0]).to(torch.float8_e4m3fn).view(torch.uint8)
                  .item(), dtype=np.uint8)
    out = A.sparse_attention(np.zeros((64, 512)), one, idx, two, t=300, swa_pos0=250)
    assert np.allclose(out, (7 * 3.0 + 40 * 2.0) / 47, rtol=0, atol=1e-6)
    # a window buffer that starts after the window: only the selected rows
    out = A.sparse_attention(np.zeros((64, 512)), one, idx, two, t=300, swa_pos0=301)
    assert np.allclose(out, 3.0, rtol=0, atol=0)


def _token_rows(tokens):
    # window row of token tok: the E4M3 value (tok mod 16) / 4 in every channel
    v = torch.tensor([(int(x) % 16) / 4.0 for x in tokens]).to(torch.float8_e4m3fn)
    return np.repeat(v.view(torch.uint8).numpy()[:, None], 512, axis=1)


def test_ring_window_equals_linear_window():
    # appending tokens 0..t one at a time into row tok mod S of a ring holds the
    # same window as a linear buffer of the last S tokens
    rng = np.random.default_rng(24)
    cache = _rand_cache(rng, 900)
    idx = np.sort(rng.choice(900, 512, replace=False)).astype(np.int32)
    q = rng.standard_normal((64, 512)) / np.sqrt(512)
    for S, t in ((128, 127), (128, 128), (128, 1000), (160, 1000), (200, 150), (130, 5)):
        ring = np.zeros((S, 512), dtype=np.uint8)
        for tok in range(t + 1):
            ring[tok % S] = _token_rows([tok])[0]
        pos0 = max(0, t - S + 1)
        lin = _token_rows(range(pos0, pos0 + S))
        a = A.sparse_attention(q, cache, idx, ring, t=t, swa_pos0=pos0, ring=True)
        b = A.sparse_attention(q, cache, idx, lin, t=t, swa_pos0=pos0)
        assert np.array_equal(a, b), (S, t)
        toks, rows = A.window_rows(t, pos0, S, ring=True)
        assert toks.tolist() == list(range(max(0, t - 127), t + 1))
        assert rows.tolist() == [x % S for x in toks.tolist()]


def test_ring_window_closed_form_names_the_tokens_used():
    # with no selected rows and a zero query the output is the mean of the
    # window rows' values (tok mod 16) / 4 over exactly the held window tokens
    S = 128
    ring = np.zeros((S, 512), dtype=np.uint8)
    t = 1000
    for tok in range(t + 1):
        ring[tok % S] = _token_rows([tok])[0]
    idx = np.full(512, -1, dtype=np.int32)
    out = A.sparse_attention(np.zeros((64, 512)), _rand_cache(np.random.default_rng(0), 4), idx,
                             ring, t=t, swa_pos0=t - S + 1, ring=True)
    want = np.mean([(x % 16) / 4.0 for x in range(t - 127, t + 1)])
    assert np.allclose(out, want, rtol=0, atol=1e-6)
    # the oldest held token is t - 100: only tokens t-100..t count
    out = A.sparse_attention(np.zeros((64, 512)), _rand_cache(np.random.default_rng(0), 4), idx,
                             ring, t=t, swa_pos0=t - 100, ring=True)
    want = np.mean([(x % 16) / 4.0 for x in range(t - 100, t + 1)])
    assert np.allclose(out, want, rtol=0, atol=1e-6)
