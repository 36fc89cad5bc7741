"""Pins for the oracle's PDM draft path and PDM prefill, against an independent route.

The oracle steps a pipeline: each step it re-encodes the PDM window (rows pdm_len ..
newest) one row at a time against its persistent PDM KV. The reference here steps
nothing (tests/reference_torch.py): for a step it takes the token sequence 0 .. newest,
runs one causal forward of the target to get every depth of every position, builds each
row's feature at the depth the row has when the PDM reads it (depth L for positions
that have left the pipeline, the stage start for in-flight ones; one stage deeper under
output-state speculation), and runs one causal forward of the PDM over all rows, with
the PDM's own final norm and the tied head on the newest row (pith.science review,
"What carries the argument" and "Core claim"). Every RMSNorm gain is drawn at random
(1 + 0.25 N(0, 1)), so a gain applied to the wrong vector shows.

Pinned: each step's draft logits, the PDM KV rows the oracle keeps for good (the
verified prefix at full depth), and the PDM prefill's KV. Three plausible mistakes are
planted in copies of the oracle's PDM pass (a RoPE position and KV slot one off, the
target's final norm on the newest row, a window that starts at the oldest in-flight
token) and each must fail these checks.
"""
import numpy as np
import pytest

import reference_torch as ref
from conftest import workload
from oracle.sampling import Sampling
from oracle.spd import SPD

LOGIT_ATOL = 1e-8


def random_gains(W, seed=7):
    rng = np.random.default_rng(seed)
    out = dict(W)
    for k, a in W.items():
        if k.endswith("norm"):
            out[k] = (1.0 + 0.25 * rng.standard_normal(a.shape)).astype(np.float32)
    return out


def read_depths(spd, newest, after_step):
    """Depth of every position 0 .. newest when the PDM reads it this step."""
    depth = [spd.L] * (newest + 1)
    for pos, st in spd.F:
        depth[pos] = int(spd.starts[st] + (spd.sizes[st] if after_step else 0))
    return depth


def reference_step(spd, cfg, W, after_step):
    newest = spd.F[-1][0]
    toks = [spd.tok[x] for x in range(newest + 1)]
    Hs = ref.target_depths(cfg, W, toks)
    X = ref.features(cfg, Hs, read_depths(spd, newest, after_step), spd.B, spd.fill)
    return ref.pdm_forward(cfg, W, X, spd.Ls)


def assert_kv_rows(spd, kv, rows, where):
    for r, (K, V) in enumerate(kv):
        np.testing.assert_allclose(spd.m.pdm.K[r][:rows], K[:rows].numpy(), rtol=1e-9, atol=1e-12,
                                   err_msg=f"{where}: PDM layer {r} K")
        np.testing.assert_allclose(spd.m.pdm.V[r][:rows], V[:rows].numpy(), rtol=1e-9, atol=1e-12,
                                   err_msg=f"{where}: PDM layer {r} V")


def check_pdm(cls, name, plen, steps, T=1.0, seed=3, fill="clamp", speculate_from="input"):
    """Runs `cls` (the oracle, or a copy with a planted mistake) and checks the prefill's
    PDM KV, then every step's draft logits and the PDM KV rows it keeps for good."""
    cfg, W, prompt = workload(name)
    W = random_gains(W)
    prompt = prompt[:plen]
    after = speculate_from == "output"
    spd = cls(cfg, W, Sampling(temperature=T, seed=seed), fill=fill, speculate_from=speculate_from)
    spd.prefill(prompt)
    Hs = ref.target_depths(cfg, W, prompt)
    X = ref.features(cfg, Hs, [cfg.n_layers] * plen, spd.B, fill)
    _, kv = ref.pdm_forward(cfg, W, X, spd.Ls)
    assert_kv_rows(spd, kv, plen, "prefill")
    outcomes = set()
    for k in range(steps):
        z_ref, kv = reference_step(spd, cfg, W, after)
        rec = spd.step()
        err = float(np.abs(rec.draft_logits - z_ref).max())
        assert err <= LOGIT_ATOL, f"step {k + 1}: draft logits differ by {err}"
        assert_kv_rows(spd, kv, spd.pdm_len, f"step {k + 1}")
        if rec.exited:
            outcomes.add(rec.accepted)
    return outcomes


# (workload, prompt length, steps, sampling seed): seeds whose T=1 runs hold both accepts
# and rejects within the checked steps
CASES = [("tiny", 32, 10, 4), ("mid_bf16_L6_d384_n3", 48, 12, 3),
         ("mid_hybrid_bf16_L8_d256_n4", 40, 15, 3)]


@pytest.mark.parametrize("name,plen,steps,seed", CASES)
def test_draft_logits_and_pdm_kv_match_independent_route(name, plen, steps, seed):
    outcomes = check_pdm(SPD, name, plen, steps, seed=seed)
    assert outcomes == {True, False}, "the checked steps should hold accepts and rejects"


@pytest.mark.parametrize("name,plen,steps,seed", CASES[:2])
def test_output_state_drafts_match_independent_route(name, plen, steps, seed):
    check_pdm(SPD, name, plen, steps, seed=seed, speculate_from="output")


def test_zero_fill_and_greedy_drafts_match_independent_route():
    check_pdm(SPD, "tiny", 32, 8, fill="zero")
    check_pdm(SPD, "mid_bf16_L7_d256_n3_uneven", 45, 10, T=0.0)


# ---- planted mistakes: each must fail the pin ------------------------------------------

class ShiftedPositions(SPD):
    """The PDM layers run each window row at position x + 1 (RoPE and KV slot)."""

    def pdm_pass(self, newest):
        m, L = self.m, self.L
        rows = list(range(self.pdm_len, newest + 1))
        depths = [self.depth.get(x, L) for x in rows]
        Z = {x: self.feature(x) for x in rows}
        for r in range(self.Ls):
            for x in rows:
                Z[x] = m.pdm.decode_layer(r, Z[x], x + 1)
        return rows, depths, m.logits(Z[newest], "pdm.final_norm")


class TargetFinalNorm(SPD):
    """The newest row is normalised with the target's final gain, not the PDM's own."""

    def pdm_pass(self, newest):
        m, L = self.m, self.L
        rows = list(range(self.pdm_len, newest + 1))
        depths = [self.depth.get(x, L) for x in rows]
        Z = {x: self.feature(x) for x in rows}
        for r in range(self.Ls):
            for x in rows:
                Z[x] = m.pdm.decode_layer(r, Z[x], x)
        return rows, depths, m.logits(Z[newest], "final_norm")


class WindowAtOldestInFlight(SPD):
    """The window starts at the oldest in-flight token, so the rows that have just left the
    pipeline never get their full-depth PDM KV."""

    def pdm_pass(self, newest):
        m, L = self.m, self.L
        rows = list(range(self.F[0][0], newest + 1))
        depths = [self.depth.get(x, L) for x in rows]
        Z = {x: self.feature(x) for x in rows}
        for r in range(self.Ls):
            for x in rows:
                Z[x] = m.pdm.decode_layer(r, Z[x], x)
        return rows, depths, m.logits(Z[newest], "pdm.final_norm")


@pytest.mark.parametrize("cls", [ShiftedPositions, TargetFinalNorm, WindowAtOldestInFlight])
@pytest.mark.parametrize("name,plen,steps,seed", [CASES[0], CASES[1]])
def test_planted_pdm_mistakes_fail_the_pin(cls, name, plen, steps, seed):
    with pytest.raises(AssertionError):
        check_pdm(cls, name, plen, steps, seed=seed)
