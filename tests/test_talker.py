"""The Talker decode step: oracle pins (CPU) and GPU parity.

The oracle (oracle/talker.py) is pinned to:
  * brute force: cached decode steps from an empty history equal the whole
    sequence recomputed with explicit loops and an explicit causal mask;
  * cache consistency: the history written by earlier steps, fed back as a
    history, reproduces the later steps;
  * the zero-layer closed form: H = output_norm * x / rms(x), logits = head . H;
  * the bf16 rounding of the cache: hand-worked values at and around the
    rounding midpoints.
  * an independent implementation of the same block: transformers' dense
    Qwen3 decoder stack (input RMSNorm, q/k/v with per-head q/k RMSNorm and
    rotate-half RoPE, GQA, output projection, post-attention RMSNorm, SwiGLU,
    final norm) loaded with the same weights, over whole sequences, and the
    predictor oracle's block step (itself pinned to transformers' code
    predictor) fed the same layer weights.  The pages give the Talker the
    predictor's block tensors (rightkit-qts exporter README, "Loader
    contract"), so a swapped gate/up, a misplaced q/k norm or a wrong GQA
    grouping in the Talker step fails here.
GPU parity compares the HIP path with the oracle on the same seeded weights,
histories and inputs.
"""
import dataclasses
import math

import numpy as np
import pytest

from oracle import talker as TK
from rvq_codebook_code_amd import synth


def _tiny(**over):
    wl = synth.TALKER_WORKLOADS["talker_tiny"]
    g = dataclasses.replace(wl.geom, **over)
    return wl, g, synth.make_talker_weights(g, wl.weight_seed)


def test_bf16_rounding_hand_values():
    one = 1.0
    ulp = 2.0 ** -7                               # bf16 spacing in [1, 2)
    cases = [(1.0, 1.0), (one + ulp / 2, 1.0),   # midpoint, even neighbour below
             (one + 3 * ulp / 2, one + 2 * ulp),  # midpoint, even neighbour above
             (one + ulp / 2 + 2.0 ** -20, one + ulp), (-(one + ulp / 2 + 2.0 ** -20), -(one + ulp)),
             (3.0e-3, 0.0030059814453125), (0.0, 0.0)]
    for x, want in cases:
        assert TK.bf16_round(np.array([x]))[0] == want, (x, want)


@pytest.mark.parametrize("kv_round", [False, True])
def test_cached_steps_equal_full_sequence(kv_round):
    wl, g, W = _tiny()
    model = TK.TalkerOracle(W, g)
    X = synth.make_talker_inputs(g, 1, 6, 11)[:, 0]
    empty = np.zeros((g.n_layers, 0, g.n_kv_heads, g.head_dim))
    steps = TK.run_steps(model, X, 0, empty, empty, kv_round=kv_round)
    full = TK.forward_full(model, X, kv_round=kv_round)
    got = np.stack([r["H"] for r in steps])
    # bf16 rounding of keys computed in two orders may, very rarely, land on
    # different sides of a midpoint; exact arithmetic agrees to 1e-12
    tol = 1e-12 if not kv_round else 1e-6
    assert np.abs(got - full).max() <= tol


def test_history_written_by_steps_reproduces_later_steps():
    wl, g, W = _tiny()
    model = TK.TalkerOracle(W, g)
    K0, V0 = synth.make_talker_history(g, 7, 21)
    K0 = TK.bf16_round(synth_bits_to_f64(K0))
    V0 = TK.bf16_round(synth_bits_to_f64(V0))
    X = synth.make_talker_inputs(g, 1, 5, 12)[:, 0]
    whole = TK.run_steps(model, X, 7, K0, V0)
    first = TK.run_steps(model, X[:3], 7, K0, V0)
    K1 = np.concatenate([K0, np.stack([r["k_new"] for r in first], axis=1)], axis=1)
    V1 = np.concatenate([V0, np.stack([r["v_new"] for r in first], axis=1)], axis=1)
    rest = TK.run_steps(model, X[3:], 10, K1, V1)
    for a, b in zip(whole[3:], rest):
        np.testing.assert_array_equal(a["H"], b["H"])
        assert a["q0"] == b["q0"]


def test_zero_layers_closed_form():
    wl, g, W = _tiny(n_layers=0)
    model = TK.TalkerOracle(W, g)
    x = synth.make_talker_inputs(g, 1, 1, 13)[0, 0].astype(np.float64)
    empty = np.zeros((0, 0, g.n_kv_heads, g.head_dim))
    r = TK.decode_step(model, x, 0, empty, empty)
    gain = W["output_norm"].astype(np.float64)
    H = gain * x / np.sqrt(np.mean(x * x) + g.rms_eps)
    np.testing.assert_allclose(r["H"], H, rtol=0, atol=1e-12)
    head = np.array([[synth_bits_to_f64(w) for w in row] for row in W["codec_head"][:5]])
    np.testing.assert_allclose(r["logits"][:5], head @ H, rtol=0, atol=1e-12)


def _library_talker(model, g):
    """transformers' dense Qwen3 decoder stack with the oracle's (materialised)
    weights, float64, eager attention."""
    import torch
    from transformers.models.qwen3.configuration_qwen3 import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3Model
    cfg = Qwen3Config(vocab_size=8, hidden_size=g.d_model, intermediate_size=g.d_ffn,
                      num_hidden_layers=g.n_layers, num_attention_heads=g.n_q_heads,
                      num_key_value_heads=g.n_kv_heads, head_dim=g.head_dim, rms_norm_eps=g.rms_eps,
                      rope_parameters={"rope_type": "default", "rope_theta": g.rope_base},
                      attention_bias=False, use_sliding_window=False, max_position_embeddings=4096)
    cfg._attn_implementation = "eager"
    m = Qwen3Model(cfg).double().eval()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    with torch.no_grad():
        for li in range(g.n_layers):
            lw, L = model.layer(li), m.layers[li]
            L.input_layernorm.weight.copy_(T(lw["attn_norm"]))
            L.post_attention_layernorm.weight.copy_(T(lw["ffn_norm"]))
            L.self_attn.q_proj.weight.copy_(T(lw["wq"]))
            L.self_attn.k_proj.weight.copy_(T(lw["wk"]))
            L.self_attn.v_proj.weight.copy_(T(lw["wv"]))
            L.self_attn.o_proj.weight.copy_(T(lw["wo"]))
            L.self_attn.q_norm.weight.copy_(T(lw["q_norm"]))
            L.self_attn.k_norm.weight.copy_(T(lw["k_norm"]))
            L.mlp.gate_proj.weight.copy_(T(lw["w_gate"]))
            L.mlp.up_proj.weight.copy_(T(lw["w_up"]))
            L.mlp.down_proj.weight.copy_(T(lw["w_down"]))
        m.norm.weight.copy_(T(model.output_norm))
    return m


@pytest.mark.parametrize("which", ["tiny", "l2_widths"])
def test_decode_steps_match_library_qwen3_stack(which):
    """Cached decode steps from an empty history (exact cache values) against
    transformers' Qwen3 decoder stack run over the whole sequence: H at every
    position, and the codec head's logits of that H."""
    import torch
    if which == "tiny":
        wl, g, W = _tiny()
        n = 6
    else:
        wl = synth.TALKER_WORKLOADS["talker_l2"]
        g = dataclasses.replace(wl.geom, n_layers=1, d_ffn=1024, vocab=64)
        W = synth.make_talker_weights(g, 3101)
        n = 4
    model = TK.TalkerOracle(W, g)
    X = synth.make_talker_inputs(g, 1, n, 31)[:, 0].astype(np.float64)
    empty = np.zeros((g.n_layers, 0, g.n_kv_heads, g.head_dim))
    steps = TK.run_steps(model, X, 0, empty, empty, kv_round=False)
    lib = _library_talker(model, g)
    with torch.no_grad():
        ref = lib(inputs_embeds=torch.from_numpy(X[None]), use_cache=False).last_hidden_state[0].numpy()
    got = np.stack([r["H"] for r in steps])
    # the library builds its RoPE table in fp32 (about 4e-7 here); a wrong
    # block (a swapped gate/up, a misplaced q/k norm) moves H by O(1)
    err = np.abs(got - ref).max()
    assert err <= 1e-5, err
    lg = np.stack([r["logits"] for r in steps])
    np.testing.assert_allclose(lg, ref @ model.head.T, rtol=0, atol=1e-5)


def test_decode_step_block_equals_predictor_block():
    """One Talker step against the predictor oracle's block step on the same
    layer weights (the predictor's decode_position is pinned to transformers'
    code predictor): from an exact history written by earlier positions, the
    residual stream after the stack, normed with the output gain, is H."""
    from oracle import predictor as PO
    wl, g, W = _tiny()
    model = TK.TalkerOracle(W, g)
    n = 5
    X = synth.make_talker_inputs(g, 1, n, 41)[:, 0].astype(np.float64)
    empty = np.zeros((g.n_layers, 0, g.n_kv_heads, g.head_dim))
    steps = TK.run_steps(model, X, 0, empty, empty, kv_round=False)

    class _PredView:     # the predictor oracle reads .g and .layers only
        pass
    pv = _PredView()
    pv.g = g
    pv.layers = [model.layer(l) for l in range(g.n_layers)]
    kc = np.zeros((g.n_layers, 1, n, g.n_kv_heads, g.head_dim))
    vc = np.zeros_like(kc)
    for pos in range(n):
        x = PO.decode_position(pv, X[pos][None], pos, kc, vc)[0]
        H = PO.rms_norm(x, model.output_norm, g.rms_eps)
        assert np.abs(H - steps[pos]["H"]).max() <= 1e-12
        np.testing.assert_allclose(steps[pos]["k_new"], kc[:, 0, pos], rtol=0, atol=1e-12)
        np.testing.assert_allclose(steps[pos]["v_new"], vc[:, 0, pos], rtol=0, atol=1e-12)


def synth_bits_to_f64(bits):
    """bf16 bit patterns to float64, written out here (not the oracle's
    helper) so the closed form above is checked by a second route."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# GPU parity through the C ABI
# ----------------------------------------------------------------------------

MARGIN = 0.05       # q0 compared where the oracle's top-2 logit gap exceeds it


def tol_for(n_layers):
    """Bar for H and logits: the bf16 bar of the predictor (3e-2 at its 5
    layers), scaled by sqrt(depth / 5).  Every layer rounds its product
    operands, the attention output and the SwiGLU output to bf16; the
    rounding errors are independent and add in quadrature, so the drift grows
    as sqrt(depth).  (An oracle run that rounds at the same places drifts by
    8.7e-3, 1.9e-2 and 3.6e-2 from the exact one at 2, 8 and 28 layers of the
    1.7B widths.)"""
    return 3e-2 * math.sqrt(max(n_layers, 5) / 5.0)


def _torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def _bits_to_dev(torch, dev, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def _run_and_compare(name, model, tk, geom, slots, hist, X, max_batch_rows=None, keep_layers=True):
    """Load each row's history into its slot, run the steps on the GPU and
    compare every step with the oracle run from the same history."""
    torch, dev = _torch_dev()
    from rvq_codebook_code_amd import binding as bd  # noqa: F401
    B = len(slots)
    steps = X.shape[0]
    for b in range(B):
        K, V = hist[b]
        if K.shape[1]:
            tk.load_history(int(slots[b]), _bits_to_dev(torch, dev, K), _bits_to_dev(torch, dev, V))
    n0 = np.array([hist[b][0].shape[1] for b in range(B)])
    st = torch.from_numpy(np.asarray(slots, dtype=np.int32)).to(dev)
    H = torch.full((B, geom.d_model), float("nan"), device=dev)
    q0 = torch.full((B,), -1, dtype=torch.int32, device=dev)
    lg = torch.full((B, geom.vocab), float("nan"), device=dev)
    got = []
    for i in range(steps):
        pos = n0 + i
        pt = torch.from_numpy(pos.astype(np.int32)).to(dev)
        tk.step(torch.from_numpy(np.ascontiguousarray(X[i])).to(dev), st, pt, int(pos.max()) + 1, H, q0, lg)
        torch.cuda.synchronize()
        got.append((H.cpu().numpy().copy(), q0.cpu().numpy().copy(), lg.cpu().numpy().copy()))
    assert tk.get_error() == 0
    worst_h = worst_l = 0.0
    agree = sure_n = 0
    for b in range(B):
        K = synth_bits_to_f64(hist[b][0])
        V = synth_bits_to_f64(hist[b][1])
        ref = TK.run_steps(model, X[:, b].astype(np.float64), int(n0[b]), K, V)
        for i in range(steps):
            h_err = np.abs(got[i][0][b] - ref[i]["H"]).max()
            l_err = np.abs(got[i][2][b] - ref[i]["logits"]).max()
            worst_h, worst_l = max(worst_h, h_err), max(worst_l, l_err)
            if ref[i]["margin"] > MARGIN:
                sure_n += 1
                agree += int(got[i][1][b] == ref[i]["q0"])
                assert got[i][1][b] == ref[i]["q0"], (name, b, i)
    tol = tol_for(geom.n_layers)
    print(f"[{name}] H max-abs {worst_h:.3g} logits max-abs {worst_l:.3g} (bar {tol:.3g}) "
          f"q0 decisive {sure_n}/{B * steps}")
    assert worst_h <= tol and worst_l <= tol
    return got


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["talker_tiny", "talker_tiny_q8", "talker_tiny_q4", "talker_wide", "talker_l2"])
def test_talker_steps_against_oracle(name):
    """Rows in permuted slots with histories of different lengths (empty,
    short, several attention splits), three consecutive steps each; bf16,
    Q8_0 and Q4_0 weights (the quantised codes enter the products exactly,
    as on the predictor's batched path); and a width above 2048, where the
    products' RMSNorm row sums and the final kernel's row take more than one
    group of loads."""
    _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS[name]
    g = wl.geom
    W = synth.make_talker_weights(g, wl.weight_seed)
    model = TK.TalkerOracle(W, g)
    lens = [0, 5, 37, wl.context] if name == "talker_l2" else [0, 3, 17, wl.context]
    slots = [3, 0, 5, 1]
    hist = [synth.make_talker_history(g, n, wl.input_seed + 10 + b) for b, n in enumerate(lens)]
    X = synth.make_talker_inputs(g, len(slots), 3, wl.input_seed)
    tk = bd.Talker(W, g, max_batch=8, n_slots=6, max_ctx=wl.context + 8)
    _run_and_compare(name, model, tk, g, slots, hist, X)
    tk.close()


@pytest.mark.gpu
def test_talker_last_position():
    """Steps up to the last position a slot holds (max_ctx - 1 = 129: three
    64-position chunks, the split count rounded up to four), then one more
    step, which raises the position flag."""
    torch, dev = _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS["talker_tiny"]
    g = wl.geom
    W = synth.make_talker_weights(g, wl.weight_seed)
    model = TK.TalkerOracle(W, g)
    tk = bd.Talker(W, g, max_batch=2, n_slots=2, max_ctx=130)
    hist = [synth.make_talker_history(g, 127, 81), synth.make_talker_history(g, 60, 82)]
    X = synth.make_talker_inputs(g, 2, 3, 83)
    _run_and_compare("talker last position", model, tk, g, [1, 0], hist, X)
    H = torch.zeros((1, g.d_model), device=dev)
    q0 = torch.zeros((1,), dtype=torch.int32, device=dev)
    tk.step(torch.from_numpy(X[0][:1]).to(dev), torch.tensor([1], dtype=torch.int32, device=dev),
            torch.tensor([130], dtype=torch.int32, device=dev), 130, H, q0)
    assert tk.get_error() & 1
    tk.close()


@pytest.mark.gpu
def test_talker_zero_layers():
    """Degenerate Talker without blocks: H is the output norm of the input
    row and q0 the head's argmax (the oracle's zero-layer closed form); the
    histories are empty tensors."""
    _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS["talker_tiny"]
    g = dataclasses.replace(wl.geom, n_layers=0)
    W = synth.make_talker_weights(g, wl.weight_seed)
    model = TK.TalkerOracle(W, g)
    hist = [synth.make_talker_history(g, n, 70 + n) for n in (0, 3)]
    X = synth.make_talker_inputs(g, 2, 2, 71)
    tk = bd.Talker(W, g, max_batch=4, n_slots=4, max_ctx=16)
    _run_and_compare("talker L=0", model, tk, g, [1, 3], hist, X)
    tk.close()


@pytest.mark.gpu
def test_talker_flags_and_cache_untouched():
    """A row with a position beyond the attention grid that max_len sizes
    (chunks of at least 64 positions), past max_ctx, negative, or an unknown
    slot raises its flag and writes nothing: a later valid step still
    matches the oracle."""
    torch, dev = _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS["talker_tiny"]
    g = wl.geom
    W = synth.make_talker_weights(g, wl.weight_seed)
    model = TK.TalkerOracle(W, g)
    tk = bd.Talker(W, g, max_batch=4, n_slots=4, max_ctx=200)
    K, V = synth.make_talker_history(g, 20, 77)
    tk.load_history(2, _bits_to_dev(torch, dev, K), _bits_to_dev(torch, dev, V))
    x = torch.from_numpy(synth.make_talker_inputs(g, 1, 1, 5)[0]).to(dev)
    H = torch.zeros((1, g.d_model), device=dev)
    q0 = torch.zeros((1,), dtype=torch.int32, device=dev)
    for slot, pos, bit in [(2, 100, 1), (2, 200, 1), (9, 20, 2), (-1, 20, 2), (2, -3, 1)]:
        tk.step(x, torch.tensor([slot], dtype=torch.int32, device=dev), torch.tensor([pos], dtype=torch.int32, device=dev),
                21, H, q0)
        assert tk.get_error() & bit
    with pytest.raises(bd.QpError):
        tk.step(x, torch.tensor([2], dtype=torch.int32, device=dev), torch.tensor([20], dtype=torch.int32, device=dev),
                201, H, q0)
    X = synth.make_talker_inputs(g, 1, 2, 6)
    _run_and_compare("talker_tiny after flags", model, tk, g, [2], [(K, V)], X)
    tk.close()


@pytest.mark.gpu
def test_talker_full_depth_rows():
    """The 1.7B Talker (28 layers) on two rows, 1 and 700 positions of
    history, one step, against the oracle run layer by layer."""
    _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS["talker_b1"]
    g = wl.geom
    W = synth.make_talker_weights(g, wl.weight_seed)
    model = TK.TalkerOracle(W, g, keep=False)
    hist = [synth.make_talker_history(g, n, 901 + n) for n in (1, 700)]
    X = synth.make_talker_inputs(g, 2, 1, 902)
    tk = bd.Talker(W, g, max_batch=2, n_slots=2, max_ctx=704)
    _run_and_compare("talker 1.7B", model, tk, g, [1, 0], hist, X)
    tk.close()


@pytest.mark.gpu
def test_talker_full_size_batch_from_graph():
    """The configuration the bench times: the 1.7B Talker, B = 16 requests
    with 1,024 positions of history each, one step replayed from a graph (no
    logits hook).  Rows 0 and 15 (own histories; the other rows share a third
    one) against the oracle: H within the depth-scaled bar, q0 where the
    oracle's top-2 gap is decisive."""
    torch, dev = _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS["talker_b16"]
    g, B, ctx = wl.geom, wl.batch, wl.context
    W = synth.make_talker_weights(g, wl.weight_seed)
    model = TK.TalkerOracle(W, g, keep=False)
    tk = bd.Talker(W, g, max_batch=B, n_slots=B, max_ctx=ctx + 8)
    own = {0: synth.make_talker_history(g, ctx, 911), B - 1: synth.make_talker_history(g, ctx, 912)}
    shared = synth.make_talker_history(g, ctx, 913)
    for b in range(B):
        K, V = own.get(b, shared)
        tk.load_history(b, _bits_to_dev(torch, dev, K), _bits_to_dev(torch, dev, V))
    X = synth.make_talker_inputs(g, B, 1, 914)[0]
    H = torch.full((B, g.d_model), float("nan"), device=dev)
    q0 = torch.full((B,), -1, dtype=torch.int32, device=dev)
    tk.step(torch.from_numpy(np.ascontiguousarray(X)).to(dev), torch.arange(B, dtype=torch.int32, device=dev),
            torch.full((B,), ctx, dtype=torch.int32, device=dev), ctx + 1, H, q0)
    torch.cuda.synchronize()
    assert tk.get_error() == 0
    Hg, qg = H.cpu().numpy(), q0.cpu().numpy()
    tol = tol_for(g.n_layers)
    for b, (K, V) in own.items():
        ref = TK.decode_step(model, X[b].astype(np.float64), ctx, synth_bits_to_f64(K), synth_bits_to_f64(V))
        err = np.abs(Hg[b] - ref["H"]).max()
        print(f"[talker B=16 graph] row {b} H max-abs {err:.3g} (bar {tol:.3g}) margin {ref['margin']:.3g}")
        assert err <= tol
        if ref["margin"] > MARGIN:
            assert qg[b] == ref["q0"]
    tk.close()


@pytest.mark.gpu
def test_talker_graph_replays_equal_direct_launches():
    """Steps replayed from graphs (no logits hook) equal the directly
    launched ones bit for bit, as the history grows across split-count
    buckets and the batch size changes."""
    torch, dev = _torch_dev()
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS["talker_tiny"]
    g = wl.geom
    W = synth.make_talker_weights(g, wl.weight_seed)
    tk = bd.Talker(W, g, max_batch=4, n_slots=8, max_ctx=160)
    lens = [29, 60, 3, 0]
    for b, n in enumerate(lens):
        K, V = synth.make_talker_history(g, n, 300 + b)
        if n:
            for base in (0, 4):                   # the same history in slots b and b + 4
                tk.load_history(b + base, _bits_to_dev(torch, dev, K), _bits_to_dev(torch, dev, V))
    X = synth.make_talker_inputs(g, 4, 40, 301)
    for i in range(40):
        B = 4 if i % 7 else 2
        pos = np.array(lens[:B]) + i
        xs = torch.from_numpy(np.ascontiguousarray(X[i, :B])).to(dev)
        pt = torch.from_numpy(pos.astype(np.int32)).to(dev)
        outs = []
        for base, with_logits in ((0, True), (4, False)):
            st = torch.arange(base, base + B, dtype=torch.int32, device=dev)
            H = torch.zeros((B, g.d_model), device=dev)
            q0 = torch.zeros((B,), dtype=torch.int32, device=dev)
            lg = torch.zeros((B, g.vocab), device=dev) if with_logits else None
            tk.step(xs, st, pt, int(pos.max()) + 1, H, q0, lg)
            torch.cuda.synchronize()
            outs.append((H.cpu().numpy(), q0.cpu().numpy()))
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
    # (rows 2 and 3 skip the steps with B = 2, leaving cleared positions in
    # their history; both slot sets skip the same ones)
    assert tk.get_error() == 0
    tk.close()
