"""Speculative generation loops over the C ABI (the workloads' drivers).

One round [first page, Algorithm 1; fifth page, the speculative_step sketch]:
the drafter proposes gamma tokens, then ``spec_decode_step`` verifies them in
one target pass, samples, and commits the target cache.  The host reads n and
the emitted tokens once per round (stop test, n-gram lookup, bookkeeping).

Drafters:
  * ModelDrafter -- a draft model (a separate small model, or the target's
    first layers: the self-speculative variant of the fifth page).  It keeps
    its own KV cache and re-feeds the last two committed tokens each round
    (its length is first rewound to the target's length - 1), then samples
    x_i ~ q_i with ``spec_reject_sample(gamma=0)``, all on the device.
  * NgramDrafter -- prompt lookup on the host [second page, "The three
    proposers"]; its proposals are one-hot, so q is NULL.
  * DeviceNgramDrafter -- the same lookup on the device, for graph-replayed
    rounds with no host round trip.
Plain decoding (the speed baseline) is ``spec_decode_step`` with gamma = 0.
"""

from __future__ import annotations

import time
from typing import Optional

import numpy as np
import torch

from synth import round_uniforms

from . import binding as bd


def _dev_i32(a) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def ngram_lookup(context, n: int, gamma: int, n_max: Optional[int] = None) -> list:
    """Tokens that followed the most recent earlier occurrence of the last k
    context tokens (up to gamma of them), for the longest k in [n, n_max]
    (n_max defaults to n) that occurs; [] when none does."""
    ctx = list(context)
    L = len(ctx)
    for k in range(n if n_max is None else n_max, n - 1, -1):
        if gamma <= 0 or L < k + 1:
            continue
        key = ctx[L - k:]
        for start in range(L - k - 1, -1, -1):
            if ctx[start:start + k] == key:
                return ctx[start + k:start + k + gamma]
    return []


class ModelDrafter:
    kind = "model"

    def __init__(self, model: bd.SpecModel, B: int, gamma: int, max_ctx: int, temperature: float = 1.0):
        self.model, self.B, self.gamma, self.T = model, B, gamma, temperature
        V = model.shape.vocab
        self.kv = bd.KVCache(model.shape, model.n_layers, B, max_ctx)
        self.ws2 = bd.workspace(model.workspace_bytes(B, 2, max_ctx))
        self.ws1 = bd.workspace(model.workspace_bytes(B, 1, max_ctx))
        self.sws = bd.workspace(bd.spec_sampler_workspace_bytes(2 * B, B, V))
        self.logits2 = torch.empty((B, 2, V), dtype=torch.float32, device="cuda")
        self.probs2 = torch.empty_like(self.logits2)
        self.logits1 = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
        self.qtmp = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
        self.q = torch.empty((B, gamma, V), dtype=torch.float32, device="cuda")
        self.drafts = torch.empty((B, gamma), dtype=torch.int32, device="cuda")
        self.x = torch.empty((B, 1), dtype=torch.int32, device="cuda")
        self.n_tmp = torch.empty(B, dtype=torch.int32, device="cuda")

    def prefill(self, prompt: np.ndarray):
        B, P = prompt.shape
        if P > 1:
            ws = bd.workspace(self.model.workspace_bytes(B, P - 1, self.kv.max_ctx))
            bd.spec_verify_forward(self.model, self.kv, B, P - 1, _dev_i32(prompt[:, :-1]), None, ws)
            bd.spec_kv_set_len(self.kv, B, None, P - 1)

    def draft(self, tok2: torch.Tensor, target_len: torch.Tensor, u_draft: torch.Tensor):
        """tok2 [B, 2] = (previous, last) committed tokens; u_draft [gamma, B].
        Returns (drafts [B, gamma] int32, q [B, gamma, V] float32, n_draft None)."""
        B, V = self.B, self.model.shape.vocab
        bd.spec_kv_set_len(self.kv, B, target_len, -1)
        bd.spec_verify_forward(self.model, self.kv, B, 2, tok2, self.logits2, self.ws2)
        bd.spec_kv_set_len(self.kv, B, None, 2)
        if B == 1:
            # one sequence: the q rows, the drawn tokens and the second
            # logits row are contiguous slices, so the kernels write them in
            # place (no copies, and the first softmax covers one row)
            bd.spec_softmax_pq(self.logits2[:, 1], 1, V, self.T, self.q[:, 0], self.sws)
            for i in range(self.gamma):
                if i > 0:
                    bd.spec_verify_forward(self.model, self.kv, 1, 1, self.drafts[:, i - 1:i], self.logits1,
                                           self.ws1)
                    bd.spec_kv_set_len(self.kv, 1, None, 1)
                    bd.spec_softmax_pq(self.logits1, 1, V, self.T, self.q[:, i], self.sws)
                bd.spec_reject_sample(1, 0, V, self.q[:, i], None, None, None, None, u_draft[i], self.n_tmp,
                                      self.drafts[:, i:i + 1], self.sws)
            return self.drafts, self.q, None
        bd.spec_softmax_pq(self.logits2, 2 * B, V, self.T, self.probs2, self.sws)
        self.qtmp.copy_(self.probs2[:, 1:2])
        for i in range(self.gamma):
            if i > 0:
                bd.spec_verify_forward(self.model, self.kv, B, 1, self.x, self.logits1, self.ws1)
                bd.spec_kv_set_len(self.kv, B, None, 1)
                bd.spec_softmax_pq(self.logits1, B, V, self.T, self.qtmp, self.sws)
            bd.spec_reject_sample(B, 0, V, self.qtmp, None, None, None, None, u_draft[i], self.n_tmp, self.x,
                                  self.sws)
            self.q[:, i].copy_(self.qtmp[:, 0])
            self.drafts[:, i].copy_(self.x[:, 0])
        return self.drafts, self.q, None


class NgramDrafter:
    """Prompt lookup with match lengths n_max down to n (n_max defaults to n).
    ``fill`` supplies gamma tokens when the lookup proposes fewer (so every
    round verifies B x (gamma+1) rows); the strict hit count is kept either
    way."""

    kind = "ngram"

    def __init__(self, B: int, gamma: int, n: int = 3, fill=None, n_max: Optional[int] = None):
        self.B, self.gamma, self.n, self.fill = B, gamma, n, fill
        self.n_max = n if n_max is None else n_max
        self.hits = 0
        self.lookups = 0

    def propose(self, contexts):
        g = self.gamma
        drafts = np.zeros((self.B, g), dtype=np.int32)
        nd = np.zeros(self.B, dtype=np.int32)
        for b, ctx in enumerate(contexts):
            prop = ngram_lookup(ctx, self.n, g, self.n_max)
            self.lookups += 1
            self.hits += bool(prop)
            if len(prop) < g and self.fill is not None:
                prop = list(prop) + list(self.fill(b, len(ctx), g - len(prop)))
            nd[b] = len(prop)
            drafts[b, :len(prop)] = prop
        return drafts, nd


class DeviceNgramDrafter:
    """Prompt lookup on the device (``spec_ngram_propose``) for graph-replayed
    rounds: the context is everything committed before the generation started
    plus the tokens the rounds append on the device; match lengths n_max down
    to n, as NgramDrafter.  ``fill_off`` [B] (optional) pads short proposals
    with the committed prefix from that offset, as NgramDrafter's ``fill``
    does with a prompt offset."""

    kind = "ngram-device"

    def __init__(self, B: int, gamma: int, n: int = 3, fill_off=None, n_max: Optional[int] = None):
        self.B, self.gamma, self.n = B, gamma, n
        self.n_max = n if n_max is None else n_max
        self.fill_off = None if fill_off is None else _dev_i32(fill_off)
        self.drafts = torch.empty((B, max(gamma, 1)), dtype=torch.int32, device="cuda")
        self.n_draft = torch.empty(B, dtype=torch.int32, device="cuda")
        self.n_found = torch.empty(B, dtype=torch.int32, device="cuda")

    def bind(self, committed, out, out_len, cap: int):
        """Set the context: committed [B] lists (the prefix rows) and the
        device buffers the rounds append to."""
        P = max(len(c) for c in committed)
        rows = np.zeros((self.B, P), dtype=np.int32)
        for b, c in enumerate(committed):
            rows[b, :len(c)] = c
        self.prefix = _dev_i32(rows)
        self.prefix_len = _dev_i32([len(c) for c in committed])
        self.P, self.out, self.out_len, self.cap = P, out, out_len, cap

    def propose(self):
        bd.spec_ngram_propose(self.B, self.n, self.n_max, self.gamma, self.prefix, self.prefix_len, self.P, self.out,
                              self.out_len, self.cap, self.fill_off, self.drafts, self.n_draft, self.n_found)
        return self.drafts, self.n_draft


class SpecDecoder:
    """B sequences of speculative decoding with one target model."""

    def __init__(self, target: bd.SpecModel, B: int, gamma: int, max_ctx: int, drafter=None,
                 temperature: float = 1.0, seed: int = 0):
        self.target, self.B, self.gamma, self.T, self.seed = target, B, gamma, temperature, seed
        V = target.shape.vocab
        self.kv = bd.KVCache(target.shape, target.n_layers, B, max_ctx)
        self.ws = bd.workspace(target.workspace_bytes(B, gamma + 1, max_ctx))
        self.drafter = drafter
        self.n = torch.empty(B, dtype=torch.int32, device="cuda")
        self.emitted = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
        self.last = torch.empty(B, dtype=torch.int32, device="cuda")
        self.tok2 = torch.empty((B, 2), dtype=torch.int32, device="cuda")
        self.V = V
        self.committed = None

    def prefill(self, prompt: np.ndarray):
        B, P = prompt.shape
        if P > 1:
            ws = bd.workspace(self.target.workspace_bytes(B, P - 1, self.kv.max_ctx))
            bd.spec_verify_forward(self.target, self.kv, B, P - 1, _dev_i32(prompt[:, :-1]), None, ws)
            bd.spec_kv_set_len(self.kv, B, None, P - 1)
        if isinstance(self.drafter, ModelDrafter):
            self.drafter.prefill(prompt)
        self.committed = [list(map(int, prompt[b])) for b in range(B)]
        self.prompt_len = P

    def _uniforms(self, r: int):
        u = round_uniforms(self.seed, r, self.B, self.gamma)
        return (torch.as_tensor(u["u_acc"]).cuda(), torch.as_tensor(u["u_res"]).cuda(),
                torch.as_tensor(np.ascontiguousarray(u["u_draft"].T)).cuda())

    def round(self, r: int, uniforms=None, logits_out=None):
        """One speculative round; returns (n [B], emitted [B, gamma+1]) on the host.
        ``logits_out`` [B, gamma+1, V] float32 receives the verify logits when given."""
        B, g = self.B, self.gamma
        u_acc, u_res, u_draft = uniforms if uniforms is not None else self._uniforms(r)
        self.last.copy_(torch.as_tensor(np.array([c[-1] for c in self.committed], np.int32)), non_blocking=False)
        q = nd = drafts = None
        if g > 0:
            if isinstance(self.drafter, ModelDrafter):
                pairs = np.array([[c[-2], c[-1]] for c in self.committed], np.int32)
                self.tok2.copy_(torch.as_tensor(pairs))
                drafts, q, nd = self.drafter.draft(self.tok2, self.kv.len, u_draft)
            else:
                d_host, nd_host = self.drafter.propose(self.committed)
                drafts, nd = _dev_i32(d_host), _dev_i32(nd_host)
        self.last_round = (drafts, q, nd)  # this round's draft inputs, for inspection
        bd.spec_decode_step(self.target, self.kv, B, g, self.T, self.last, drafts, nd, q, u_acc if g else None,
                            u_res, self.n, self.emitted, logits_out, self.ws)
        n = self.n.cpu().numpy()
        em = self.emitted.cpu().numpy()
        for b in range(B):
            self.committed[b] += [int(t) for t in em[b, :n[b] + 1]]
        return n, em

    def generate(self, n_new: int, preload_uniforms: bool = True) -> dict:
        """Rounds until every sequence has n_new new tokens (then truncated)."""
        B, g = self.B, self.gamma
        max_rounds = n_new + 1
        pool = [self._uniforms(r) for r in range(max_rounds)] if preload_uniforms else None
        torch.cuda.synchronize()
        accepted_per_pos = np.zeros(max(g, 1), dtype=np.int64)
        rounds, accepted, t0 = 0, 0, time.perf_counter()
        round_ms = []
        while min(len(c) for c in self.committed) - self.prompt_len < n_new:
            t1 = time.perf_counter()
            n, _ = self.round(rounds, pool[rounds] if pool else None)
            round_ms.append((time.perf_counter() - t1) * 1e3)
            accepted += int(n.sum())
            for i in range(g):
                accepted_per_pos[i] += int((n > i).sum())
            rounds += 1
        wall = time.perf_counter() - t0
        tokens = [c[self.prompt_len:self.prompt_len + n_new] for c in self.committed]
        num_drafts = rounds * B
        return {
            "tokens": tokens, "rounds": rounds, "wall_s": wall, "tok_s": B * n_new / wall,
            "accepted": accepted, "drafted": num_drafts * g, "num_drafts": num_drafts,
            "mean_acceptance_length": 1.0 + accepted / num_drafts,
            "acceptance_rate": accepted / max(num_drafts * g, 1),
            "per_position": (accepted_per_pos / num_drafts).tolist() if g else [],
            "round_ms_p50": float(np.percentile(round_ms, 50)), "round_ms_p99": float(np.percentile(round_ms, 99)),
        }

    def generate_graph(self, n_new: int) -> dict:
        """The rounds of generate(), with the same uniforms, run as replays of
        one captured HIP graph per round: the drafter's passes, the verify
        step and the round bookkeeping (spec_commit_round) all stay on the
        device.  Per round the host only copies that round's uniforms into the
        graph's buffers; it reads the output count once per batch of rounds,
        each batch no longer than the fewest rounds that could finish."""
        B, g = self.B, self.gamma
        if g > 0 and not isinstance(self.drafter, (ModelDrafter, DeviceNgramDrafter)):
            raise ValueError("graph rounds need a device drafter (ModelDrafter, DeviceNgramDrafter) or gamma = 0")
        cap = n_new + g + 1
        dev = "cuda"
        tok2 = _dev_i32([[c[-2], c[-1]] for c in self.committed])
        last = _dev_i32([c[-1] for c in self.committed])
        out = torch.zeros((B, cap), dtype=torch.int32, device=dev)
        out_len = torch.zeros(B, dtype=torch.int32, device=dev)
        max_rounds = n_new + 1
        pool = [self._uniforms(r) for r in range(max_rounds)]
        ua_all = torch.stack([p[0] for p in pool]) if g else None
        ur_all = torch.stack([p[1] for p in pool])
        ud_all = torch.stack([p[2] for p in pool]) if g else None
        u_acc = torch.empty_like(ua_all[0]) if g else None
        u_res = torch.empty_like(ur_all[0])
        u_draft = torch.empty_like(ud_all[0]) if g else None

        def load_uniforms(r):
            if g:
                u_acc.copy_(ua_all[r])
                u_draft.copy_(ud_all[r])
            u_res.copy_(ur_all[r])

        ngram = isinstance(self.drafter, DeviceNgramDrafter)
        if ngram:
            self.drafter.bind(self.committed, out, out_len, cap)

        def body():
            drafts = q = nd = None
            if g and ngram:
                drafts, nd = self.drafter.propose()
            elif g:
                drafts, q, _ = self.drafter.draft(tok2, self.kv.len, u_draft)
            bd.spec_decode_step(self.target, self.kv, B, g, self.T, last, drafts, nd, q, u_acc, u_res, self.n,
                                self.emitted, None, self.ws)
            bd.spec_commit_round(B, g, self.n, self.emitted, tok2, last, out, out_len, cap)

        # Round 0 runs eagerly (it also performs every kernel's one-time
        # set-up) and is timed; the capture that follows records the round
        # without running it and is not timed, as a server captures once.
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        load_uniforms(0)
        body()
        torch.cuda.synchronize()
        wall0 = time.perf_counter() - t0
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            body()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rounds = 1
        while True:
            remaining = n_new - int(out_len.min().item())
            if remaining <= 0:
                break
            for _ in range(max(1, -(-remaining // (g + 1)))):
                load_uniforms(rounds)
                graph.replay()
                rounds += 1
        torch.cuda.synchronize()
        wall = wall0 + time.perf_counter() - t0
        total = out_len.cpu().numpy()
        toks = out.cpu().numpy()
        tokens = [list(map(int, toks[b, :n_new])) for b in range(B)]
        for b in range(B):
            self.committed[b] += list(map(int, toks[b, :min(int(total[b]), cap)]))
        accepted = int(total.sum()) - rounds * B
        return {"tokens": tokens, "rounds": rounds, "wall_s": wall, "tok_s": B * n_new / wall,
                "mean_acceptance_length": 1.0 + accepted / (rounds * B),
                "acceptance_rate": accepted / max(rounds * B * g, 1)}

