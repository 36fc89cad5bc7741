"""HIP path vs oracle, step by step, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest

from conftest import workload
from parity import run_parity

pytestmark = pytest.mark.gpu

_dev = {}


def dev_weights(name):
    if name not in _dev:
        import torch
        from speculative_pipeline_decoding_amd import upload_weights
        cfg, W, _ = workload(name)
        _dev.clear()
        torch.cuda.empty_cache()
        _dev[name] = upload_weights(cfg, W)
    return _dev[name]


def _run(name, **kw):
    cfg, W, prompt = workload(name)
    print(f"[parity] {name} {kw}", flush=True)
    rep = run_parity(cfg, W, dev_weights(name), prompt, **kw)
    print(f"[parity] {name} {kw} -> {rep}", flush=True)
    return rep


def test_tiny_greedy_full_length():
    rep = _run("tiny")
    assert rep["stopped_at_near_tie"] is None and rep["N"] == 63


def test_tiny_sampled():
    rep = _run("tiny", T=1.0, seed=3)
    assert rep["steps"] > 0


@pytest.mark.parametrize("n", [1, 3, 4])
def test_tiny_other_widths(n):
    rep = _run("tiny", n=n, G=30)
    assert rep["steps"] > 0


def test_tiny_forced_and_zero_fill():
    from oracle.spd import ar_decode
    cfg, W, prompt = workload("tiny")
    ref = ar_decode(cfg, W, prompt, G=cfg.gen_len + 8)
    rep = _run("tiny", forced_p=0.7, forced_ref=ref, seed=5, fill="zero")
    assert rep["stopped_at_near_tie"] is None


@pytest.mark.parametrize("name", ["mid_bf16_L6_d384_n3", "mid_bf16_L7_d256_n3_uneven",
                                  "mid_f32_L4_d128_n1", "mid_bf16_L4_d512_hd128_n4",
                                  "mid_hybrid_bf16_L8_d256_n4"])
def test_mid_greedy(name):
    rep = _run(name)
    assert rep["steps"] > 0


@pytest.mark.parametrize("name", ["mid_bf16_L6_d384_n3", "mid_bf16_L4_d512_hd128_n4",
                                  "mid_hybrid_bf16_L8_d256_n4"])
def test_mid_sampled(name):
    rep = _run(name, T=1.0, seed=7)
    assert rep["steps"] > 0


@pytest.mark.parametrize("top_p,T,seed", [(0.875, 1.0, 3), (0.25, 0.7, 4)])
def test_tiny_top_p(top_p, T, seed):
    rep = _run("tiny", T=T, seed=seed, top_p=top_p, slack=1e-5)
    assert rep["steps"] > 0 and rep["top_p_sets"] > rep["steps"]


def test_tiny_top_p_tied_logits():
    """LM-head rows duplicated in pairs: every logit row is made of exact ties, and the
    top-p edge often splits a pair, so the lower-id rule decides membership."""
    import torch
    from speculative_pipeline_decoding_amd import upload_weights
    cfg, W, prompt = workload("tiny")
    W2 = dict(W)
    lm = np.array(W["lm_head"], copy=True)
    lm[1::2] = lm[0::2]
    W2["lm_head"] = lm
    _dev.clear()
    torch.cuda.empty_cache()
    dW2 = upload_weights(cfg, W2)
    print("[parity] tiny, paired LM-head rows, T=1 top_p=0.625", flush=True)
    rep = run_parity(cfg, W2, dW2, prompt, T=1.0, seed=8, top_p=0.625, slack=1e-5)
    print(f"[parity] -> {rep}", flush=True)
    assert rep["steps"] > 0 and rep["top_p_sets"] > rep["steps"]
    assert rep["top_p_split_ties"] > 0      # the lower-id rule was exercised


@pytest.mark.parametrize("name,top_p", [("mid_bf16_L6_d384_n3", 0.875),
                                         ("mid_hybrid_bf16_L8_d256_n4", 0.5)])
def test_mid_top_p(name, top_p):
    rep = _run(name, T=1.0, seed=7, top_p=top_p, slack=5e-4)
    assert rep["steps"] > 0


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_mid_hybrid_planned_uneven_split(T):
    """A split from the stage planner that the default never makes ([2, 3, 1, 2] on the
    8-layer hybrid): both sides run it, in lockstep."""
    import dataclasses
    from speculative_pipeline_decoding_amd import balance_stages
    name = "mid_hybrid_bf16_L8_d256_n4"
    cfg, W, prompt = workload(name)
    sizes = balance_stages([3, 1, 1, 1, 2, 2, 1, 1], cfg.n_stages)
    assert sizes == [2, 3, 1, 2]
    cfg2 = dataclasses.replace(cfg, stage_layers=tuple(sizes))
    print(f"[parity] {name} stages {sizes} T={T}", flush=True)
    rep = run_parity(cfg2, W, dev_weights(name), prompt, T=T, seed=9)
    print(f"[parity] -> {rep}", flush=True)
    assert rep["steps"] > 0


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_wide_ffn_down_projection_on_split_k(T):
    """An FFN wider than the rows kernel's LDS stage (16904 fp32 inputs to the down
    projection, 66 KiB) runs that GEMV on the split-K kernel; lockstep with the oracle."""
    import dataclasses
    import torch
    from spd_inputs import get, make_prompt, make_weights
    from speculative_pipeline_decoding_amd import upload_weights
    cfg = dataclasses.replace(get("mid_bf16_L7_d256_n3_uneven"), name="mid_bf16_L7_d256_ffn16904",
                              d_ffn=16904)
    W = make_weights(cfg)
    prompt = make_prompt(cfg)
    _dev.clear()
    torch.cuda.empty_cache()
    print(f"[parity] {cfg.name} T={T}", flush=True)
    rep = run_parity(cfg, W, upload_weights(cfg, W), prompt, T=T, seed=5)
    print(f"[parity] -> {rep}", flush=True)
    assert rep["steps"] > 0


@pytest.mark.parametrize("name,T", [("tiny", 0.0), ("tiny", 1.0), ("mid_bf16_L6_d384_n3", 0.0),
                                    ("mid_bf16_L6_d384_n3", 1.0), ("mid_hybrid_bf16_L8_d256_n4", 1.0)])
def test_non_unit_norm_gains(name, T):
    """Every RMSNorm gain drawn as 1 + 0.25 N(0, 1) (the synthetic weights use gains of 1,
    under which a gain applied to the wrong row or vector goes unseen): lockstep with the
    oracle, including the head sweep that normalises the exiting token with the target's
    final gain and the PDM's newest row with its own."""
    import torch
    from speculative_pipeline_decoding_amd import upload_weights
    cfg, W, prompt = workload(name)
    rng = np.random.default_rng(123)
    W2 = {k: ((1.0 + 0.25 * rng.standard_normal(v.shape)).astype(np.float32) if k.endswith("norm")
              else v) for k, v in W.items()}
    assert sum(1 for k in W2 if k.endswith("norm")) >= 2 * cfg.n_layers + 2
    _dev.clear()
    torch.cuda.empty_cache()
    print(f"[parity] {name} random gains T={T}", flush=True)
    rep = run_parity(cfg, W2, upload_weights(cfg, W2), prompt, T=T, seed=3)
    print(f"[parity] -> {rep}", flush=True)
    assert rep["steps"] > 0


def test_layer_timing_single_token_passes():
    """At n = 1 every sub-layer launch serves one layer: each layer gets one timed pass
    per step, with a positive kernel time."""
    from speculative_pipeline_decoding_amd import SPD
    cfg, W, prompt = workload("mid_hybrid_bf16_L8_d256_n4")
    streams = []
    for serial in (True, None):
        gpu = SPD(cfg, dev_weights("mid_hybrid_bf16_L8_d256_n4"), n=1)
        toks = [gpu.prefill(prompt)]
        if serial:
            gpu.timing(True, serial=True)    # the PDM chain on the caller's stream
        for _ in range(6):
            gpu.step()
            toks.append(gpu.verify_commit().token)
        if serial:
            ms, passes = gpu.timing_read_layers()
        gpu.close()
        streams.append(toks)
    assert streams[0] == streams[1]          # one stream or two: the same tokens
    print(f"[timing] per-layer us per pass {np.round(1e3 * ms / np.maximum(passes, 1), 1)}",
          flush=True)
    assert passes.tolist() == [6] * cfg.n_layers
    assert np.all(ms > 0)


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("tiny", {"T": 1.0, "seed": 3}),
                                     ("tiny", {"n": 1, "G": 30}),
                                     ("mid_bf16_L6_d384_n3", {}),
                                     ("mid_bf16_L6_d384_n3", {"T": 1.0, "seed": 7}),
                                     ("mid_hybrid_bf16_L8_d256_n4", {}),
                                     ("mid_bf16_L7_d256_n3_uneven", {"T": 1.0, "seed": 2})])
def test_output_state_speculation(name, kw):
    """The PDM after the step's target layers, on their output states (the ablation of
    the early start): lockstep with the oracle in the same mode."""
    rep = _run(name, speculate_from="output", **kw)
    assert rep["steps"] > 0


def test_output_state_speculation_forced_rollbacks():
    from oracle.spd import ar_decode
    cfg, W, prompt = workload("mid_hybrid_bf16_L8_d256_n4")
    ref = ar_decode(cfg, W, prompt, G=cfg.gen_len + 8)
    rep = _run("mid_hybrid_bf16_L8_d256_n4", forced_p=0.5, forced_ref=ref, seed=4,
               speculate_from="output")
    assert rep["stopped_at_near_tie"] is None and rep["rejected"] > 2


@pytest.mark.parametrize("name,kw", [
    ("tiny", {"prompt_len": 1}),                                   # a one-token prompt
    ("tiny", {"prompt_len": 1, "T": 1.0, "seed": 2}),
    ("tiny", {"anchors": (0,)}),                                   # k = 1: the embedding only
    ("tiny", {"n": 4, "G": 30}),                                   # n = L: one layer per stage
    ("mid_bf16_L6_d384_n3", {"anchors": (0, 6), "Ls": 1, "T": 1.0, "seed": 4}),
    ("mid_bf16_L7_d256_n3_uneven", {"Ls": 3, "n": 2}),             # Ls > L / n
])
def test_degenerate_shapes(name, kw):
    import dataclasses
    import torch
    from spd_inputs import make_weights
    from speculative_pipeline_decoding_amd import upload_weights
    cfg, W, prompt = workload(name)
    kw = dict(kw)
    P = kw.pop("prompt_len", len(prompt))
    if "anchors" in kw:
        # another anchor count changes the projection's width: a model of its own
        cfg = dataclasses.replace(cfg, anchors=kw.pop("anchors"))
        W = make_weights(cfg)
        _dev.clear()
        torch.cuda.empty_cache()
        dW = upload_weights(cfg, W)
    else:
        dW = dev_weights(name)
    print(f"[parity] {name} anchors {cfg.anchors} prompt {P} {kw}", flush=True)
    rep = run_parity(cfg, W, dW, prompt[:P], **kw)
    print(f"[parity] -> steps {rep['steps']} N {rep.get('N')} err {rep['max_logit_err']:.2e}",
          flush=True)
    assert rep["steps"] > 0


@pytest.mark.parametrize("kw", [{}, {"T": 1.0, "seed": 6}, "forced"])
def test_maximum_sizes(kw):
    """The library's largest pipeline: n = 16 stages of one layer, k = 8 anchors, and n + 1
    = 17 PDM window rows (past the matrix-core GEMV's 16 columns: the split-K kernel)."""
    import dataclasses
    import torch
    from oracle.spd import ar_decode
    from spd_inputs import get, make_prompt, make_weights
    from speculative_pipeline_decoding_amd import upload_weights
    cfg = dataclasses.replace(get("mid_bf16_L7_d256_n3_uneven"), name="max_bf16_L16_d256_n16",
                              n_layers=16, n_stages=16, anchors=(0, 1, 2, 4, 6, 9, 12, 16),
                              pdm_layers=2, prompt_len=40, gen_len=14, max_ctx=96)
    W = make_weights(cfg)
    prompt = make_prompt(cfg)
    if kw == "forced":
        kw = {"forced_p": 0.75, "forced_ref": ar_decode(cfg, W, prompt, G=cfg.gen_len + 20),
              "seed": 8}
    _dev.clear()
    torch.cuda.empty_cache()
    print(f"[parity] {cfg.name} {sorted(kw)}", flush=True)
    rep = run_parity(cfg, W, upload_weights(cfg, W), prompt, **kw)
    print(f"[parity] -> steps {rep['steps']} N {rep.get('N')} rejected {rep.get('rejected')} "
          f"err {rep['max_logit_err']:.2e}", flush=True)
    assert rep["steps"] >= cfg.n_stages


def test_mid_forced_acceptance():
    from oracle.spd import ar_decode
    cfg, W, prompt = workload("mid_bf16_L6_d384_n3")
    ref = ar_decode(cfg, W, prompt, G=cfg.gen_len + 8)
    rep = _run("mid_bf16_L6_d384_n3", forced_p=0.8, forced_ref=ref, seed=2)
    assert rep["stopped_at_near_tie"] is None


def test_hybrid_rollback_restores_linear_state():
    """Frequent rejections: every reseed must continue from the linear states saved at v - 1."""
    from oracle.spd import ar_decode
    cfg, W, prompt = workload("mid_hybrid_bf16_L8_d256_n4")
    ref = ar_decode(cfg, W, prompt, G=cfg.gen_len + 8)
    rep = _run("mid_hybrid_bf16_L8_d256_n4", forced_p=0.4, forced_ref=ref, seed=4)
    assert rep["stopped_at_near_tie"] is None and rep["rejected"] > 3


def test_determinism_same_seed_same_bits():
    from speculative_pipeline_decoding_amd import SPD
    cfg, W, prompt = workload("mid_bf16_L6_d384_n3")
    outs = []
    for _ in range(2):
        g = SPD(cfg, dev_weights("mid_bf16_L6_d384_n3"), temperature=1.0, seed=11)
        toks, recs = g.generate(prompt, 16)
        outs.append((toks, g.debug("target_logits").tobytes(), g.debug("anchors").tobytes()))
        g.close()
    assert outs[0] == outs[1]


def _records(name, lookahead, G, **kw):
    """Every commit record, KV length and counter of one run through the C ABI."""
    from speculative_pipeline_decoding_amd import SPD
    cfg, W, prompt = workload(name)
    g = SPD(cfg, dev_weights(name), **kw)
    g.lookahead(lookahead)
    toks = [g.prefill(prompt)]
    recs = []
    while len(toks) < G:
        g.step()
        c = g.verify_commit()
        kv, pl = g.kv_lens()
        recs.append((c.verified, c.position, c.token, c.accepted, c.draft_token, c.flags,
                     c.committed_total, c.inflight, c.new_draft, c.newest, tuple(kv), pl))
        if c.verified:
            toks.append(c.token)
    st = g.stats()
    logits = g.debug("target_logits").tobytes()   # synchronises: no step runs ahead of it now
    g.close()
    return toks, recs, (st.K, st.N, st.accepted, st.rejected), logits


def _forced(name, p, seed):
    from oracle.spd import ar_decode
    cfg, W, prompt = workload(name)
    return dict(forced_p=p, forced_ref=ar_decode(cfg, W, prompt, G=cfg.gen_len + 8), seed=seed)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tiny", dict(temperature=1.0, seed=3)),
    ("tiny", dict(n=4, temperature=0.7, top_p=0.875, seed=1)),
    ("mid_bf16_L6_d384_n3", dict(temperature=1.0, seed=7)),
    ("mid_hybrid_bf16_L8_d256_n4", {}),
    ("mid_hybrid_bf16_L8_d256_n4", "forced"),
])
def test_lookahead_bit_identical(name, kw):
    """Launching each refill step's successor with it changes when work runs, not what it
    computes: every record, KV length, counter and the last logits match bit for bit."""
    if kw == "forced":
        kw = _forced(name, 0.4, 4)   # frequent rejections: lookahead stops at every verification
    cfg, W, prompt = workload(name)
    G = min(cfg.gen_len, 40)
    print(f"[lookahead] {name} {sorted(k for k in kw)}", flush=True)
    a = _records(name, False, G, **kw)
    b = _records(name, True, G, **kw)
    assert a[0] == b[0] and a[1] == b[1] and a[2] == b[2] and a[3] == b[3]
    if name == "tiny" and not kw:
        from oracle.spd import ar_decode
        assert b[0] == ar_decode(cfg, W, prompt, G=G)   # lossless: greedy decode of the target


def test_lookahead_reset_and_timing_guard():
    """A step launched ahead is drained by spd_reset; timing cannot start under it."""
    from speculative_pipeline_decoding_amd import SPD, SpdError
    from speculative_pipeline_decoding_amd.binding import SPD_E_STATE
    cfg, W, prompt = workload("tiny")
    ref = _records("tiny", False, 24)[0]
    g = SPD(cfg, dev_weights("tiny"))
    g.lookahead(True)
    g.prefill(prompt)
    g.step()                 # a refill step (n = 2): its successor is enqueued with it
    g.verify_commit()
    with pytest.raises(SpdError) as e:
        g.timing(True)
    assert e.value.code == SPD_E_STATE
    g.reset()
    toks = [g.prefill(prompt)]
    while len(toks) < 24:
        g.step()
        c = g.verify_commit()
        if c.verified:
            toks.append(c.token)
    g.close()
    assert toks == ref


def test_call_order_and_capacity_errors():
    from speculative_pipeline_decoding_amd import SPD, SpdError
    from speculative_pipeline_decoding_amd.binding import SPD_E_STATE, SPD_E_CAPACITY, SPD_E_ARG
    cfg, W, prompt = workload("tiny")
    g = SPD(cfg, dev_weights("tiny"))
    with pytest.raises(SpdError) as e:
        g.step()
    assert e.value.code == SPD_E_STATE
    with pytest.raises(SpdError) as e:
        g.prefill([cfg.vocab])
    assert e.value.code == SPD_E_ARG
    with pytest.raises(SpdError) as e:
        g.prefill([1] * cfg.max_ctx)
    assert e.value.code == SPD_E_CAPACITY
    g.prefill(prompt)
    with pytest.raises(SpdError) as e:
        g.prefill(prompt)
    assert e.value.code == SPD_E_STATE
    with pytest.raises(SpdError) as e:
        g.verify_commit()
    assert e.value.code == SPD_E_STATE
    g.step()
    with pytest.raises(SpdError) as e:
        g.step()
    assert e.value.code == SPD_E_STATE
    g.verify_commit()
    # run until the newest position reaches max_ctx
    with pytest.raises(SpdError) as e:
        for _ in range(4 * cfg.max_ctx):
            g.step()
            g.verify_commit()
    assert e.value.code == SPD_E_CAPACITY
    g.reset()
    assert g.prefill(prompt) >= 0
    g.close()


def test_prompt_longer_than_one_staging_piece():
    """A prompt of 132100 ids crosses the 512 KiB (131072-id) pieces in which spd_prefill
    uploads it. The K row layer 0 stores at position p depends only on the token at p and
    on p (RMSNorm, the K rows of W_qkv, RoPE at p), so the oracle's arithmetic gives it
    exactly; positions on both sides of the piece boundary, and the first and last, must
    hold the library's K rows for the right tokens."""
    import torch
    from oracle.model import Model
    from oracle.numerics import apply_rope, rmsnorm
    from speculative_pipeline_decoding_amd import SPD, upload_weights
    cfg0, W, _ = workload("tiny")
    P = 132100
    cfg = cfg0.with_(max_ctx=P + 100)
    prompt = np.random.default_rng(9).integers(0, cfg.vocab, P).astype(np.int32)
    _dev.clear()
    torch.cuda.empty_cache()
    print(f"[parity] {P}-token prompt on the tiny model", flush=True)
    gpu = SPD(cfg, upload_weights(cfg, W))
    gpu.prefill(prompt)
    kv = gpu.debug("target_kv").reshape(cfg.n_layers, 2, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
    gpu.close()
    m = Model(cfg, W)
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    for p in (0, 1, 131071, 131072, 131073, 131500, P - 1):
        a = rmsnorm(m.embed(prompt[p]), m.W("layers.0.attn_norm"), cfg.rms_eps)
        k = (m.W("layers.0.w_qkv") @ a)[hq * hd:(hq + hkv) * hd].reshape(hkv, hd)
        k = apply_rope(k, p, cfg.rope_theta)
        np.testing.assert_allclose(kv[0, 0, :, p, :], k, rtol=0, atol=1e-5,
                                   err_msg=f"layer-0 K row at position {p}")


@pytest.mark.parametrize("name,T,seed", [("mid_bf16_L4_d512_hd128_n4", 0.0, 0),
                                         ("mid_bf16_L4_d512_hd128_n4", 1.0, 6),
                                         ("mid_bf16_L6_d384_n3", 0.0, 0),
                                         ("mid_hybrid_bf16_L8_d256_n4", 1.0, 3)])
def test_fp32_kv_cache(name, T, seed):
    """kv_dtype "f32" with bf16 weights: the target and PDM KV caches hold fp32 keys and
    values (row-major V; head dims over 64 sum p V from whole V rows), in lockstep with the
    oracle storing fp32 too. With nothing rounded to bf16 on the way, the logits agree to
    1e-3, twenty times tighter than the bf16-KV bound."""
    cfg, W, prompt = workload(name)
    cfg32 = cfg.with_(kv_dtype="f32")
    print(f"[parity] {name} kv f32 T={T}", flush=True)
    rep = run_parity(cfg32, W, dev_weights(name), prompt, T=T, seed=seed, tol_logits=1e-3)
    print(f"[parity] -> {rep}", flush=True)
    assert rep["steps"] > 0


@pytest.mark.parametrize("name,w,kw", [
    ("tiny", 2, {}), ("tiny", 4, {}), ("tiny", 4, {"T": 1.0, "seed": 3}),
    ("tiny", 2, {"T": 1.0, "seed": 5}),
    ("mid_bf16_L6_d384_n3", 4, {"T": 1.0, "seed": 7, "G": 24}),
    ("mid_bf16_L4_d512_hd128_n4", 2, {"T": 1.0, "seed": 7, "G": 24})])
def test_draft_tree(name, w, kw):
    """W candidates per draft position: every candidate, the accepted rank, the siblings'
    states, and the adoption of accepted siblings (their rows and keys) in lockstep."""
    rep = _run(name, width=w, **kw)
    assert rep["steps"] > 0
    if rep["stopped_at_near_tie"] is None:
        assert rep["sibling_accepts"] > 0 and rep["adoptions"] > 0


def test_draft_tree_lookahead_bit_identical():
    import torch
    from speculative_pipeline_decoding_amd import SPD
    cfg, W, prompt = workload("tiny")
    runs = []
    for la in (False, True):
        g = SPD(cfg, dev_weights("tiny"), temperature=1.0, seed=3, draft_width=4)
        g.lookahead(la)
        out = [g.prefill(prompt)]
        while len(out) < cfg.gen_len:
            g.step()
            c = g.verify_commit()
            if c.verified:
                out.append((c.token, c.accepted_index))
        runs.append(out)
        g.close()
    torch.cuda.synchronize()
    assert runs[0] == runs[1]


@pytest.mark.parametrize("kw", [{}, {"T": 1.0, "seed": 6}])
def test_draft_tree_maximum_sizes(kw):
    """Draft trees at the largest pipeline: n = 16 stages of one layer with W = 4 candidates
    per position, so a target attention launch holds 64 problems (the most one launch takes),
    k = 8 anchors and 17 PDM window rows."""
    import dataclasses
    import torch
    from spd_inputs import get, make_prompt, make_weights
    from speculative_pipeline_decoding_amd import upload_weights
    cfg = dataclasses.replace(get("mid_bf16_L7_d256_n3_uneven"), name="max_bf16_L16_d256_n16",
                              n_layers=16, n_stages=16, anchors=(0, 1, 2, 4, 6, 9, 12, 16),
                              pdm_layers=2, prompt_len=40, gen_len=14, max_ctx=96)
    W = make_weights(cfg)
    prompt = make_prompt(cfg)
    _dev.clear()
    torch.cuda.empty_cache()
    print(f"[parity] {cfg.name} W=4 {sorted(kw)}", flush=True)
    rep = run_parity(cfg, W, upload_weights(cfg, W), prompt, width=4, **kw)
    print(f"[parity] -> steps {rep['steps']} N {rep.get('N')} sibling accepts "
          f"{rep['sibling_accepts']} adoptions {rep['adoptions']} err {rep['max_logit_err']:.2e}",
          flush=True)
    assert rep["steps"] >= cfg.n_stages or rep["stopped_at_near_tie"] is not None


@pytest.mark.parametrize("name,w,kw", [
    ("tiny", 4, {"prompt_len": 1}),                    # a one-token prompt
    ("tiny", 3, {"prompt_len": 1, "T": 1.0, "seed": 2}),
    ("tiny", 2, {"n": 1, "G": 30}),                    # n = 1: every exit verifies its own drafts
    ("tiny", 4, {"n": 1, "T": 1.0, "seed": 4, "G": 30}),
    ("tiny", 2, {"anchors": (0,)}),                    # k = 1
    ("mid_bf16_L7_d256_n3_uneven", 3, {"T": 1.0, "seed": 3, "G": 24}),
])
def test_draft_tree_degenerate_shapes(name, w, kw):
    import dataclasses
    import torch
    from spd_inputs import make_weights
    from speculative_pipeline_decoding_amd import upload_weights
    cfg, W, prompt = workload(name)
    kw = dict(kw)
    P = kw.pop("prompt_len", len(prompt))
    if "anchors" in kw:
        # another anchor count changes the projection's width: a model of its own
        cfg = dataclasses.replace(cfg, anchors=kw.pop("anchors"))
        W = make_weights(cfg)
        _dev.clear()
        torch.cuda.empty_cache()
        dW = upload_weights(cfg, W)
    else:
        dW = dev_weights(name)
    print(f"[parity] {name} W={w} anchors {cfg.anchors} prompt {P} {kw}", flush=True)
    rep = run_parity(cfg, W, dW, prompt[:P], width=w, **kw)
    print(f"[parity] -> {rep['steps']} steps, {rep['sibling_accepts']} sibling accepts", flush=True)
    assert rep["steps"] > 0


@pytest.mark.parametrize("w,T,d_ffn", [(3, 1.0, 16904), (4, 0.0, 4160), (4, 1.0, 9728)])
def test_draft_tree_long_down_projection_staged_in_chunks(w, T, d_ffn):
    """With 3 or 4 candidates per position the down projection's inputs (w x d_ffn fp32)
    exceed the rows kernel's LDS stage: it stages them in chunks of whole ring rounds
    (the last chunk partial, the boundary inside a pair of rounds with 4160). Lockstep with
    the oracle, siblings' states included."""
    import dataclasses
    import torch
    from spd_inputs import get, make_prompt, make_weights
    from speculative_pipeline_decoding_amd import upload_weights
    cfg = dataclasses.replace(get("mid_bf16_L7_d256_n3_uneven"),
                              name=f"mid_bf16_L7_d256_ffn{d_ffn}", d_ffn=d_ffn)
    W = make_weights(cfg)
    prompt = make_prompt(cfg)
    _dev.clear()
    torch.cuda.empty_cache()
    print(f"[parity] {cfg.name} W={w} T={T}", flush=True)
    rep = run_parity(cfg, W, upload_weights(cfg, W), prompt, T=T, seed=5, width=w, G=20)
    print(f"[parity] -> steps {rep['steps']} sibling accepts {rep['sibling_accepts']} "
          f"err {rep['max_logit_err']:.2e} state {rep['max_state_rel']:.2e}", flush=True)
    assert rep["steps"] > 0


@pytest.mark.parametrize("T,seed", [(0.0, 0), (1.0, 7)])
def test_draft_tree_with_fp32_kv_cache(T, seed):
    """Draft trees over fp32 KV caches with bf16 weights: the siblings' side rows are fp32
    too and their attention runs on the fp32 kernel (row-major V)."""
    cfg, W, prompt = workload("mid_bf16_L6_d384_n3")
    cfg32 = cfg.with_(kv_dtype="f32")
    print(f"[parity] mid_bf16_L6_d384_n3 kv f32 W=4 T={T}", flush=True)
    rep = run_parity(cfg32, W, dev_weights("mid_bf16_L6_d384_n3"), prompt, T=T, seed=seed,
                     width=4, tol_logits=1e-3, G=24)
    print(f"[parity] -> steps {rep['steps']} sibling accepts {rep['sibling_accepts']} "
          f"err {rep['max_logit_err']:.2e}", flush=True)
    assert rep["steps"] > 0
