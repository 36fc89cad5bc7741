"""Lockstep comparison of the HIP path (through the C ABI) with the CPU oracle.

Comparison rule:
  * integers bit-exact: first token, every step's draft, verified position,
    committed token, accept flag, KV length of every layer, PDM length;
  * floats: logits max-abs <= 1e-4 (f32 weights) / 5e-2 (bf16 weights);
    residual and anchor states relative L2 <= 1e-5 (f32) / 2e-2 (bf16);
  * draft trees (width > 1): every candidate of every draft position, the accepted
    candidate's rank, and the states of sibling candidates as above;
  * a token decision may differ only where the oracle flags a near-tie
    (top-2 gap < 1e-3, or |u q(d) - p(d)| < 1e-3 q(d)); the comparison stops there;
  * top_p < 1: every logit row must lie within `slack` of the oracle's (the envelope its
    near-tie flags assume); each top-p set the library reports must hold every token
    the oracle's envelope keeps for sure and nothing outside its band, and must be the
    top-p set of the library's own logits (check_top_p_set).
"""
from __future__ import annotations

import numpy as np

from oracle.sampling import Sampling, nucleus_bounds
from oracle.spd import SPD as OracleSPD

TOP_P_MASS_EPS = 1e-6     # fp32 exponentials and 2^-40 fixed-point masses


def check_top_p_set(z, cut, T, top_p, where):
    """The reported set {z > zb} + {z == zb, id <= id_cut} is the top-p set of z itself:
    a prefix of the tokens by decreasing logit (lower id first) that reaches top_p and
    does not without its last token; lse is log sum over it of exp(z / T)."""
    z = np.asarray(z, dtype=np.float32)
    zb, idc = np.float32(cut["zb"]), int(cut["id_cut"])
    ids = np.arange(z.size)
    keep = (z > zb) | ((z == zb) & (ids <= idc))
    assert np.any(z == zb) and keep.any(), f"{where}: zb {zb} is not a logit of the row"
    zd = z.astype(np.float64) / T
    w = np.exp(zd - zd.max())
    p = w / w.sum()
    order = np.lexsort((ids, -z.astype(np.float64)))
    k = int(keep.sum())
    assert keep[order[:k]].all(), f"{where}: the set is not a prefix of the order"
    mass = p[keep].sum()
    last = p[order[k - 1]]
    assert mass >= top_p - TOP_P_MASS_EPS, f"{where}: set mass {mass} < top_p {top_p}"
    assert mass - last < top_p + TOP_P_MASS_EPS, f"{where}: set not minimal ({mass - last})"
    lse = zd.max() + np.log(w[keep].sum())
    assert abs(float(cut["lse"]) - lse) <= 1e-5 * max(1.0, abs(lse)), f"{where}: lse"
    split = bool(np.any((z == zb) & ~keep))      # the edge fell inside a group of ties
    return keep, split


def check_against_envelope(keep, z_oracle, s, where):
    certain, band = nucleus_bounds(z_oracle, s.temperature, s.top_p, s.slack())
    assert keep[certain].all(), f"{where}: a token the oracle keeps for sure is left out"
    assert not (keep & ~(certain | band)).any(), f"{where}: a token outside the band is kept"


def tolerances(cfg):
    if cfg.dtype == "bf16":
        return 5e-2, 2e-2
    return 1e-4, 1e-5


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def run_parity(cfg, W, dW, prompt, G=None, T=0.0, seed=0, n=None, fill="clamp",
               forced_p=None, forced_ref=None, check_states=True, max_steps=None,
               oracle_weights=None, tol_logits=None, top_p=1.0, slack=None,
               speculate_from="input", anchors=None, Ls=None, progress_every=0, width=1):
    from speculative_pipeline_decoding_amd import SPD
    G = cfg.gen_len if G is None else G
    tol_l, tol_h = tolerances(cfg)
    if tol_logits is not None:
        tol_l = tol_logits
    s = Sampling(temperature=T, seed=seed, top_p=top_p, logit_slack=slack)
    nucleus = T > 0 and top_p < 1.0
    if nucleus:
        tol_l = min(tol_l, s.slack())
    kw = {"top_p": top_p, "speculate_from": speculate_from, "anchors": anchors, "Ls": Ls,
          "draft_width": width}
    if forced_p is not None:
        s.forced_p, s.forced_ref, s.forced_base = forced_p, np.asarray(forced_ref), len(prompt)
        kw.update(forced_p=forced_p, forced_ref=list(forced_ref))
    gpu = SPD(cfg, dW, temperature=T, seed=seed, n=n, fill=fill, **kw)
    model = None
    if oracle_weights is not None:
        from oracle.model import Model
        model = Model(cfg, W, weights=oracle_weights)
    orc = OracleSPD(cfg, W, s, n=n, fill=fill, model=model, speculate_from=speculate_from,
                    anchors=anchors, Ls=Ls, W=width)
    rep = {"steps": 0, "max_logit_err": 0.0, "max_state_rel": 0.0, "stopped_at_near_tie": None,
           "flagged": 0, "sibling_accepts": 0, "adoptions": 0}
    t0o = orc.prefill(prompt)
    t0g = gpu.prefill(prompt)
    zt = gpu.debug("target_logits")
    err = float(np.abs(zt - orc.prefill_logits).max())
    rep["max_logit_err"] = err
    assert err <= tol_l, f"prefill logits err {err}"
    rep["top_p_sets"] = rep["top_p_split_ties"] = 0
    if nucleus:
        keep, split = check_top_p_set(zt, gpu.debug("top_p")[0], T, top_p, "prefill")
        check_against_envelope(keep, orc.prefill_logits, s, "prefill")
        rep["top_p_sets"] += 1
        rep["top_p_split_ties"] += int(split)
    if t0g != t0o:
        assert orc.prefill_flag, f"first token {t0g} != {t0o} without a near tie"
        rep["stopped_at_near_tie"] = 0
        gpu.close()
        return rep
    ring = gpu.n + 1
    while 1 + orc.N < G and (max_steps is None or rep["steps"] < max_steps):
        rec = orc.step()
        gpu.step()
        c = gpu.verify_commit()
        rep["steps"] += 1
        k = rep["steps"]
        if progress_every and k % progress_every == 0:
            print(f"[parity] step {k}: committed {orc.N}, max logit err {rep['max_logit_err']:.3g}",
                  flush=True)
        assert c.newest == rec.newest, (k, c.newest, rec.newest)
        zq = gpu.debug("draft_logits")
        e = float(np.abs(zq - rec.draft_logits).max())
        rep["max_logit_err"] = max(rep["max_logit_err"], e)
        assert e <= tol_l, f"step {k}: draft logits err {e}"
        rep["flagged"] += int(rec.draft_flag) + int(rec.verify_flag)
        if nucleus:
            cuts = gpu.debug("top_p")
            dpos = rec.newest + 1
            keep, split = check_top_p_set(zq, cuts[1 + dpos % ring], T, top_p, f"step {k} draft")
            check_against_envelope(keep, rec.draft_logits, s, f"step {k} draft")
            rep["top_p_sets"] += 1
            rep["top_p_split_ties"] += int(split)
            if rec.exited:
                zt = gpu.debug("target_logits")
                keep, split = check_top_p_set(zt, cuts[0], T, top_p, f"step {k} target")
                check_against_envelope(keep, rec.target_logits, s, f"step {k} target")
                rep["top_p_sets"] += 1
                rep["top_p_split_ties"] += int(split)
        drafts = [c.new_draft]
        if width > 1:
            toks = gpu.debug("tokens").reshape(ring, width)
            drafts += [int(t) for t in toks[(rec.newest + 1) % ring, 1:]]
        if drafts != list(rec.drafts):
            assert rec.draft_flag, f"step {k}: drafts {drafts} != {rec.drafts} without a near tie"
            rep["stopped_at_near_tie"] = k
            break
        assert bool(c.verified) == rec.exited, (k, c.verified, rec.exited)
        if rec.exited:
            zt = gpu.debug("target_logits")
            e = float(np.abs(zt - rec.target_logits).max())
            rep["max_logit_err"] = max(rep["max_logit_err"], e)
            assert e <= tol_l, f"step {k}: target logits err {e}"
            assert c.position == rec.verified_pos
            assert c.draft_token == rec.verified_draft, (k, c.draft_token, rec.verified_draft)
            if (c.token != rec.committed or bool(c.accepted) != rec.accepted
                    or c.accepted_index != rec.accepted_index):
                assert rec.verify_flag, (f"step {k}: commit ({c.token}, {c.accepted_index}) != "
                                         f"({rec.committed}, {rec.accepted_index}) without a near tie")
                rep["stopped_at_near_tie"] = k
                break
            if c.accepted_index > 0:
                rep["sibling_accepts"] += 1
                if not rec.single:
                    rep["adoptions"] += 1
        kv, pl = gpu.kv_lens()
        assert kv == rec.kv_len, (k, kv, rec.kv_len)
        assert pl == rec.pdm_len, (k, pl, rec.pdm_len)
        assert c.committed_total == orc.N and c.inflight == len(orc.F)
        # a sibling adopted by this commit still sits in its own row: the next step moves it
        moved = {}
        if rec.exited and c.accepted_index > 0 and not rec.single:
            moved = {rec.verified_pos: c.accepted_index}
        if check_states:
            hr = gpu.debug("h_ring").reshape(ring, width, cfg.d_model)
            an = gpu.debug("anchors").reshape(ring, width, len(orc.B), cfg.d_model)
            # the oracle's token at x, and its sibling b, against ring row (x mod ring) W + b
            states = [((x, moved.get(x, 0)), hv, orc.anch.get(x, {})) for x, hv in orc.h.items()]
            states += [((x, b), hv, orc.sib_anch.get((x, b), {})) for (x, b), hv in orc.sib_h.items()]
            for (x, b), hv, amap in states:
                r = rel(hr[x % ring, b], hv)
                rep["max_state_rel"] = max(rep["max_state_rel"], r)
                assert r <= tol_h, f"step {k}: residual of position {x} candidate {b} rel err {r}"
                for i, av in amap.items():
                    r = rel(an[x % ring, b, i], av)
                    rep["max_state_rel"] = max(rep["max_state_rel"], r)
                    assert r <= tol_h, f"step {k}: anchor {i} of position {x}.{b} rel err {r}"
    st = gpu.stats()
    if rep["stopped_at_near_tie"] is None:
        assert (st.N, st.K, st.accepted, st.rejected) == (orc.N, orc.K, orc.accepted, orc.rejected)
        assert abs(st.s0 - orc.s0) < 1e-12
    rep.update(N=st.N, K=st.K, alpha=st.alpha, s0=st.s0, rejected=st.rejected,
               tokens_match=orc.committed)
    gpu.close()
    return rep
