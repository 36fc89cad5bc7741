"""Speculative Pipeline Decoding, one pipeline step at a time, and plain AR decoding.

Source: arXiv 2605.30852 as summarised on the pith.science review page
("What carries the argument", "Core claim", the Eq. (9) quote in the
circularity check, "Assumptions & free parameters") and the aiqbench abstract:
  * the target's L layers are cut into n stages; n tokens of one sequence are
    in flight, each in a different stage (the "depth staircase");
  * the Pipeline Draft Module (PDM) reads the pipeline's INPUT states, so it
    runs alongside the step: for each position it concatenates the hidden
    states at the anchor depths B that are already computed, projects k*d -> d,
    and runs Ls decoder layers plus the LM head to draft the next token;
  * verification is streaming: the token leaving the last stage verifies the
    next position; a rejection truncates the KV cache, flushes the pipeline
    and reseeds it;
  * alpha = N/K (committed tokens per pipeline step) and S0 = alpha * n (Eq. 9).

Readings, where the pages leave a step open:
  R1  anchor b = residual after b target layers (b = 0: embedding; b = L: last
      layer output before the final norm);
  R3  anchors not yet computed for a position are filled by the deepest one
      that is ("clamp"); zero fill is the alternative;
  R4  the PDM's only input is the projected feature;
  R5  the PDM re-encodes every not-yet-final position each step; a position
      whose depth is L becomes a permanent row of the PDM's KV cache;
  R8  uneven stages: numpy.array_split sizes (the first L mod n stages are larger);
  R9  after a reseed, one token enters per step, so n-1 steps verify nothing;
  R10 N excludes the prefill's first token; K counts every step;
  the embedding of the stage-0 token is part of the step's input state, so
  the newest PDM row sees it (depth 0).

Draft trees of width W (the review's "Assumptions & free parameters": W = 1 and 4; a
reading, since the pages describe no mechanism): each draft position carries W candidates
(sampling.select_drafts), best first. The first is the spine: the PDM's next draft
continues from it. The others are siblings: they enter the pipeline with the spine and
run the same stages at the same position, each attending over the cached positions before
it (the committed prefix and the spine's in-flight positions: its ancestors) and its own
key. When the token before them leaves the pipeline, all W are verified
(sampling.verify_tree). The spine accepted: as with W = 1. A sibling accepted: it is
adopted as the token at v (its keys and values move into the cache, its states become the
position's), every position after v (the spine's descendants) and this step's draft are
flushed, and the adopted token finishes its last stage in the next step. None accepted: the
usual reject and reseed. Positions whose token is already verified (a reseed, an adopted
sibling, a draft verified in the step that made it) carry one candidate.

Output-state speculation, the ablation the pith.science review mentions against the
input-state ("early start") schedule of its "Core claim": with speculate_from="output"
the PDM runs after the step's target layers and reads each position's states at its
depth after the step (one stage deeper; the exiting token at depth L), so it cannot
overlap the step. A position whose depth reaches L in this step becomes a permanent PDM
row in the same step. Everything else (drafting, verification, rollback) is unchanged.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from spd_inputs.configs import ModelConfig
from .model import Model
from .sampling import Sampling, first_token, select_drafts, verify_tree, argmax_lowest


def stage_sizes(L: int, n: int, explicit: Sequence[int] = ()) -> List[int]:
    """Layers per stage: explicit sizes, else numpy.array_split's split of L into n."""
    if explicit:
        sizes = list(explicit)
        assert len(sizes) == n and sum(sizes) == L and min(sizes) >= 1
        return sizes
    return [len(a) for a in np.array_split(np.arange(L), n)]


@dataclass
class StepRecord:
    K: int                       # steps so far, this one included
    newest: int                  # position of the stage-0 token this step
    draft: int                   # d, drafted for position newest + 1
    draft_flag: bool
    exited: bool
    exit_pos: int = -1
    verified_pos: int = -1       # v = exit_pos + 1
    verified_draft: int = -1     # token at v before verification
    committed: int = -1          # y
    accepted: bool = False
    verify_flag: bool = False
    target_logits: Optional[np.ndarray] = None
    draft_logits: Optional[np.ndarray] = None
    kv_len: List[int] = field(default_factory=list)
    pdm_len: int = 0
    inflight: List[Tuple[int, int]] = field(default_factory=list)
    pdm_rows: Tuple[int, int] = (0, 0)   # window [first, last] of PDM rows this step
    pdm_row_depths: List[int] = field(default_factory=list)
    drafts: List[int] = field(default_factory=list)        # the W candidates drafted this step
    verified_cands: List[int] = field(default_factory=list)  # candidates tested at v
    accepted_index: int = -1     # which candidate was accepted (-1: none)
    single: bool = False         # the exiting token was alone: v held this step's drafts


class SPD:
    """The SPD state machine on one sequence."""

    def __init__(self, cfg: ModelConfig, arrays: Dict[str, np.ndarray], sampling: Sampling,
                 n: Optional[int] = None, anchors: Optional[Sequence[int]] = None,
                 Ls: Optional[int] = None, fill: str = "clamp", ft=np.float64,
                 model: Optional[Model] = None, record_logits: bool = True,
                 speculate_from: str = "input", W: int = 1):
        assert speculate_from in ("input", "output")
        assert W >= 1
        self.W = W
        if W > 1:
            assert speculate_from == "input" and sampling.forced_p is None
            assert sampling.top_p >= 1.0 and all(k == 0 for k in cfg.kinds)
        self.output_states = speculate_from == "output"
        self.cfg = cfg
        self.n = cfg.n_stages if n is None else n
        self.B = list(cfg.anchors if anchors is None else anchors)
        self.Ls = cfg.pdm_layers if Ls is None else Ls
        assert self.B[0] == 0 and all(a < b for a, b in zip(self.B, self.B[1:]))
        assert self.B[-1] <= cfg.n_layers and 1 <= self.n <= cfg.n_layers
        assert self.Ls <= cfg.pdm_layers
        assert fill in ("clamp", "zero")
        self.fill = fill
        self.s = sampling
        self.m = model if model is not None else Model(cfg, arrays, ft)
        self.L = cfg.n_layers
        self.sizes = stage_sizes(self.L, self.n, cfg.stage_layers if n is None else ())
        self.starts = list(np.cumsum([0] + self.sizes[:-1]))
        self.record_logits = record_logits
        # state
        self.tok: Dict[int, int] = {}          # token at each position (prompt, committed, in flight)
        self.h: Dict[int, np.ndarray] = {}     # residual of positions in flight
        self.anch: Dict[int, Dict[int, np.ndarray]] = {}   # position -> anchor index -> state
        self.depth: Dict[int, int] = {}        # delta(p): target layers applied to p
        self.q: Dict[int, np.ndarray] = {}     # PDM distribution each draft was drawn from
        self.zq: Dict[int, np.ndarray] = {}    # and the logits it was computed from
        self.F: List[List[int]] = []           # in flight, oldest first: [pos, stage]
        self.kv_len = [0] * self.L
        self.pdm_len = 0
        self.N = self.K = self.accepted = self.rejected = 0
        self.committed: List[int] = []         # generated stream incl. the first token
        self.P0 = 0
        # draft tree: sibling candidates (ranks 1 .. W-1) of in-flight positions, their
        # residuals and anchor states
        self.sib: Dict[int, List[int]] = {}
        self.sib_h: Dict[Tuple[int, int], np.ndarray] = {}
        self.sib_anch: Dict[Tuple[int, int], Dict[int, np.ndarray]] = {}

    # -- prefill -------------------------------------------------------------
    def prefill(self, prompt: np.ndarray) -> int:
        m, B, L = self.m, self.B, self.L
        P0 = len(prompt)
        assert P0 >= 1
        self.P0 = P0
        for i, t in enumerate(prompt):
            self.tok[i] = int(t)
        H = m.embed_many(np.asarray(prompt))
        A: Dict[int, np.ndarray] = {0: H.copy()}
        for l in range(L):
            H = m.target.prefill_layer(l, H, 0)
            if (l + 1) in B:
                A[B.index(l + 1)] = H.copy()
        self.kv_len = [P0] * L
        z = m.logits(H[-1])
        t0, flag = first_token(z, self.s, P0)
        self.prefill_logits, self.prefill_flag = z, flag
        # PDM over the verified prefix, features at full depth
        X = np.concatenate([A[i] for i in range(len(B))], axis=1)
        Z = X @ m.W("pdm.proj").T
        for r in range(self.Ls):
            Z = m.pdm.prefill_layer(r, Z, 0)
        self.pdm_len = P0
        # reseed state with the first token at stage 0
        self.tok[P0] = t0
        self.F = [[P0, 0]]
        self.committed = [t0]
        return t0

    # -- the PDM feature of one position (anchor aggregation) ---------------------
    def feature(self, x: int) -> np.ndarray:
        d = self.m.cfg.d_model
        delta = self.depth.get(x, self.L)
        avail = [i for i, b in enumerate(self.B) if b <= delta]
        deepest = avail[-1]
        parts = []
        for i, b in enumerate(self.B):
            if b <= delta:
                parts.append(self.anch[x][i])
            elif self.fill == "clamp":
                parts.append(self.anch[x][deepest])
            else:
                parts.append(np.zeros(d, self.m.ft))
        return self.m.W("pdm.proj") @ np.concatenate(parts)

    # -- the PDM over its window ----------------------------------------------------
    def pdm_pass(self, newest: int):
        """PDM over the rows pdm_len .. newest at the depths they have now.

        Rows before the oldest in-flight position are at depth L (their features are
        final and their PDM KV rows are rewritten here once more, then kept); in-flight
        rows carry their current, partial depth. Each row runs the Ls layers at its own
        absolute position, attending over the PDM KV at positions <= its own. The newest
        row's final-normed state (the PDM's own final norm) goes through the tied head.
        Returns (rows, their depths, the newest row's logits)."""
        m, L = self.m, self.L
        rows = list(range(self.pdm_len, newest + 1))
        depths = [self.depth.get(x, L) for x in rows]
        Z = {x: self.feature(x) for x in rows}
        for r in range(self.Ls):
            for x in rows:
                Z[x] = m.pdm.decode_layer(r, Z[x], x)
        return rows, depths, m.logits(Z[newest], "pdm.final_norm")

    # -- one pipeline step ------------------------------------------------------
    def step(self) -> StepRecord:
        m, n, L, B = self.m, self.n, self.L, self.B
        newest = self.F[-1][0]
        # 1. the stage-0 token enters: embedding = anchor 0 (every step except the one after a
        #    sibling was adopted, whose newest token is the adopted one, in its last stage)
        if self.F[-1][1] == 0:
            h0 = m.embed(self.tok[newest])
            self.h[newest] = h0
            self.anch[newest] = {0: h0.copy()}
            self.depth[newest] = 0
            for b, t in enumerate(self.sib.get(newest, []), start=1):
                hs = m.embed(t)
                self.sib_h[(newest, b)] = hs
                self.sib_anch[(newest, b)] = {0: hs.copy()}
        else:
            assert self.W > 1 and len(self.F) == 1 and self.F[0][1] == n - 1
        exiting = self.F[0][1] == n - 1

        def target_pass():
            """Each in-flight token (and its sibling candidates) runs its stage's layers."""
            for pos, st in self.F:
                layers = range(self.starts[st], self.starts[st] + self.sizes[st])
                h = self.h[pos]
                for l in layers:
                    h = m.target.decode_layer(l, h, pos)
                    if (l + 1) in B:
                        self.anch[pos][B.index(l + 1)] = h.copy()
                    self.kv_len[l] = pos + 1
                self.h[pos] = h
                self.depth[pos] += self.sizes[st]
                for b in range(1, len(self.sib.get(pos, [])) + 1):
                    hs = self.sib_h[(pos, b)]
                    for l in layers:
                        hs = m.target.decode_layer(l, hs, pos, branch=b)
                        if (l + 1) in B:
                            self.sib_anch[(pos, b)][B.index(l + 1)] = hs.copy()
                    self.sib_h[(pos, b)] = hs

        if self.output_states:
            # 3, then 2: the PDM reads the states the step produced
            target_pass()
            rows, depths, z_q = self.pdm_pass(newest)
            # positions whose depth is L now (the exiting one included) become permanent
            self.pdm_len = max(self.pdm_len, self.F[0][0] + (1 if exiting else 0))
        else:
            # 2. PDM on the step's input states (early start)
            rows, depths, z_q = self.pdm_pass(newest)
            # positions whose depth is already L become permanent PDM rows
            self.pdm_len = max(self.pdm_len, self.F[0][0])
            # 3. target
            target_pass()
        dpos = newest + 1
        drafts, q, dflag = select_drafts(z_q, self.s, dpos, self.W)
        d = drafts[0]
        if q is not None:
            self.q[dpos] = q
            self.zq[dpos] = z_q
        self.K += 1
        rec = StepRecord(K=self.K, newest=newest, draft=d, draft_flag=dflag, exited=False,
                         draft_logits=z_q if self.record_logits else None,
                         pdm_rows=(rows[0], rows[-1]), pdm_row_depths=depths, drafts=drafts)
        # 4. streaming verification of the position after the exiting token
        if self.F[0][1] == n - 1:
            p = self.F[0][0]
            v = p + 1
            z_t = m.logits(self.h[p])
            single = len(self.F) == 1
            cands = drafts if single else [self.tok[v]] + self.sib.get(v, [])
            y, idx, vflag = verify_tree(z_t, cands, self.q.get(v), self.s, v)
            acc = idx >= 0
            self.N += 1
            self.committed.append(y)
            rec.exited, rec.exit_pos, rec.verified_pos = True, p, v
            rec.verified_draft, rec.committed, rec.accepted, rec.verify_flag = cands[0], y, acc, vflag
            rec.verified_cands, rec.accepted_index, rec.single = list(cands), idx, single
            rec.target_logits = z_t if self.record_logits else None
            if acc and (idx == 0 or single):
                # the spine (or, when v is this step's draft, any candidate: none of them has
                # entered the pipeline yet) is the token at v; the pipeline shifts
                self.accepted += 1
                self._drop_siblings(lambda x: x != v)
                if single:
                    self.F = [[dpos, 0]]
                    self.tok[dpos] = y
                else:
                    self.F = [[pos, st + 1] for pos, st in self.F[1:]] + [[dpos, 0]]
                    self.tok[dpos] = d
                    if len(drafts) > 1:
                        self.sib[dpos] = drafts[1:]
            elif acc:
                # a sibling at v: it becomes the token at v, and the spine's descendants go
                self.accepted += 1
                st_v = self.F[1][1]
                ran = list(range(self.starts[st_v] + self.sizes[st_v]))
                m.target.adopt(v, idx, ran)
                self.h[v] = self.sib_h[(v, idx)]
                self.anch[v] = self.sib_anch[(v, idx)]
                self.kv_len = [min(k, v + 1 if l < len(ran) else v) for l, k in enumerate(self.kv_len)]
                m.target.truncate(v + 1)
                self._forget_from(v + 1)
                self._drop_siblings(lambda x: x < v)
                self.tok[v] = y
                self.F = [[v, st_v + 1]]
            else:
                # 5. reject: truncate, flush, reseed (v, y) at stage 0
                self.rejected += 1
                self.kv_len = [min(k, v) for k in self.kv_len]
                m.target.truncate(v)
                self._forget_from(v)
                self._drop_siblings(lambda x: x < v)
                self.tok[v] = y
                self.F = [[v, 0]]
        else:
            # refill step: nothing leaves the pipeline
            self.F = [[pos, st + 1] for pos, st in self.F] + [[dpos, 0]]
            self.tok[dpos] = d
            if len(drafts) > 1:
                self.sib[dpos] = drafts[1:]
        # forget states nobody reads again
        for old in [x for x in self.h if x < self.pdm_len]:
            self.h.pop(old, None)
            self.anch.pop(old, None)
            self.depth.pop(old, None)
        for old in [x for x in self.q if x < self.pdm_len]:
            self.q.pop(old, None)
            self.zq.pop(old, None)
        self._drop_siblings(lambda x: x >= self.pdm_len)
        rec.kv_len = list(self.kv_len)
        rec.pdm_len = self.pdm_len
        rec.inflight = [tuple(f) for f in self.F]
        return rec

    # -- draft-tree bookkeeping ----------------------------------------------------
    def _forget_from(self, x0: int) -> None:
        """Drop every state and token of positions >= x0 (a flush)."""
        for dead in [x for x in self.h if x >= x0]:
            self.h.pop(dead, None)
            self.anch.pop(dead, None)
            self.depth.pop(dead, None)
        self.tok = {x: t for x, t in self.tok.items() if x < x0}
        for dead in [x for x in self.q if x >= x0]:
            self.q.pop(dead, None)
            self.zq.pop(dead, None)

    def _drop_siblings(self, keep) -> None:
        """Forget the sibling candidates (and their side keys) of positions failing keep."""
        for x in [x for x in self.sib if not keep(x)]:
            for b in range(1, len(self.sib[x]) + 1):
                self.sib_h.pop((x, b), None)
                self.sib_anch.pop((x, b), None)
            del self.sib[x]
        self.m.target.drop_side(keep)

    # -- statistics (Eq. 9) --------------------------------------------------------
    @property
    def alpha(self) -> float:
        return self.N / self.K if self.K else 0.0

    @property
    def s0(self) -> float:
        return self.alpha * self.n


@dataclass
class SpdResult:
    tokens: List[int]            # generated stream, the prefill's first token included
    records: List[StepRecord]
    N: int
    K: int
    accepted: int
    rejected: int
    alpha: float
    s0: float
    prefill_logits: np.ndarray
    prefill_flag: bool


def spd_run(cfg: ModelConfig, arrays, prompt, G: Optional[int] = None,
            sampling: Optional[Sampling] = None, **kw) -> SpdResult:
    """Prefill, then pipeline steps until G tokens (first token included) are committed."""
    G = cfg.gen_len if G is None else G
    spd = SPD(cfg, arrays, sampling or Sampling(), **kw)
    spd.prefill(np.asarray(prompt))
    recs = []
    while 1 + spd.N < G:
        recs.append(spd.step())
    return SpdResult(spd.committed, recs, spd.N, spd.K, spd.accepted, spd.rejected,
                     spd.alpha, spd.s0, spd.prefill_logits, spd.prefill_flag)


def ar_decode(cfg: ModelConfig, arrays, prompt, G: Optional[int] = None, ft=np.float64,
              model: Optional[Model] = None, return_logits: bool = False):
    """Plain greedy decoding: prefill, then each token through all L layers and argmax."""
    G = cfg.gen_len if G is None else G
    m = model if model is not None else Model(cfg, arrays, ft)
    prompt = np.asarray(prompt)
    P0 = len(prompt)
    H = m.embed_many(prompt)
    for l in range(cfg.n_layers):
        H = m.target.prefill_layer(l, H, 0)
    z = m.logits(H[-1])
    toks = [argmax_lowest(z)]
    logits = [z]
    pos = P0
    while len(toks) < G:
        h = m.embed(toks[-1])
        for l in range(cfg.n_layers):
            h = m.target.decode_layer(l, h, pos)
        z = m.logits(h)
        toks.append(argmax_lowest(z))
        logits.append(z)
        pos += 1
    return (toks, logits) if return_logits else toks
