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
  * DeviceNgramDrafter -- prompt lookup on the device [second page, "The
    three proposers"] (``spec_ngram_propose``); its proposals are one-hot,
    so q is NULL.  Eager rounds hand it the committed context each round;
    graph-replayed rounds bind it once to the device buffers the rounds
    append to.
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


def wilson_interval(k: int, n: int, z: float = 1.96) -> tuple:
    """Wilson score interval of a binomial proportion k / n."""
    if n <= 0:
        return (0.0, 1.0)
    ph = k / n
    den = 1.0 + z * z / n
    mid = (ph + z * z / (2 * n)) / den
    half = z * np.sqrt(ph * (1 - ph) / n + z * z / (4 * n * n)) / den
    return (float(max(0.0, mid - half)), float(min(1.0, mid + half)))


def acceptance_stats(n_rounds, gamma: int) -> dict:
    """Acceptance figures from the accepted lengths of every round of every
    sequence (a list of arrays), as the first page reads them off a server's
    log (section "Checking it on a real system": mean acceptance length,
    acceptance rate, per-position acceptance over the number of drafts):
      * per_position[i] = P(n >= i + 1), unconditional;
      * acceptance_rate = accepted / drafted with its 95% Wilson interval;
      * mean_acceptance_length = 1 + accepted / rounds with a 95% normal
        interval over rounds;
      * the truncated geometric fit of the i.i.d. model of the same page
        (section "Why gamma has a ceiling": P(n >= i) = alpha^i for
        i <= gamma): the maximum-likelihood alpha = sum n / (sum n +
        #{n < gamma}), and the mean acceptance length it predicts,
        (1 - alpha^(gamma + 1)) / (1 - alpha)."""
    ns = np.concatenate([np.asarray(x, np.int64).reshape(-1) for x in n_rounds]) if len(n_rounds) else np.zeros(0)
    R = int(ns.size)
    out = {"rounds_counted": R}
    if R == 0 or gamma <= 0:
        return out
    acc = int(ns.sum())
    tokens = 1.0 + ns
    sd = float(tokens.std(ddof=1)) if R > 1 else 0.0
    mal = float(tokens.mean())
    out["mean_acceptance_length"] = mal
    out["mean_acceptance_length_ci95"] = (float(mal - 1.96 * sd / np.sqrt(R)), float(mal + 1.96 * sd / np.sqrt(R)))
    out["acceptance_rate"] = acc / (R * gamma)
    out["acceptance_rate_ci95"] = wilson_interval(acc, R * gamma)
    out["per_position"] = [float((ns > i).mean()) for i in range(gamma)]
    short = int((ns < gamma).sum())
    alpha = acc / (acc + short) if acc + short > 0 else 1.0
    out["geometric_alpha"] = float(alpha)
    out["geometric_mal"] = float(gamma + 1 if alpha >= 1.0 else (1 - alpha ** (gamma + 1)) / (1 - alpha))
    return out


class ModelDrafter:
    kind = "model"

    def __init__(self, model: bd.SpecModel, B: int, gamma: int, max_ctx: int, temperature: float = 1.0):
        self.model, self.B, self.gamma, self.T = model, B, gamma, temperature
        V = model.shape.vocab
        self.kv = bd.KVCache(model.shape, model.n_layers, B, max_ctx)
        self.ws2 = bd.workspace(model.workspace_bytes(B, 2, max_ctx))
        self.ws1 = bd.workspace(model.workspace_bytes(B, 1, max_ctx))
        self.sws = bd.workspace(bd.spec_sampler_workspace_bytes(B, B, V))
        self.logits2 = torch.empty((B, 2, V), dtype=torch.float32, device="cuda")
        self.logits1 = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
        self.q = torch.empty((B, gamma, V), dtype=torch.float32, device="cuda")
        self.drafts = torch.empty((B, gamma), dtype=torch.int32, device="cuda")
        self.drafts_t = torch.empty((gamma, B), dtype=torch.int32, device="cuda")  # position-major

    def prefill(self, prompt: np.ndarray):
        B, P = prompt.shape
        if P > 1:
            ws = bd.workspace(self.model.workspace_bytes(B, P - 1, self.kv.max_ctx))
            bd.spec_verify_forward(self.model, self.kv, B, P - 1, _dev_i32(prompt[:, :-1]), None, ws)
            bd.spec_kv_set_len(self.kv, B, None, P - 1)

    def draft(self, tok2: torch.Tensor, target_len: torch.Tensor, u_draft: torch.Tensor):
        """tok2 [B, 2] = (previous, last) committed tokens; u_draft [gamma, B].
        Returns (drafts [B, gamma] int32, q [B, gamma, V] float32, n_draft None).
        Each position's sampling step writes its q rows straight into column i
        of q and its tokens into row i of the position-major drafts_t, which
        the next pass reads as its input; one transpose per round gives the
        [B, gamma] drafts (none when B = 1)."""
        B, V, g = self.B, self.model.shape.vocab, self.gamma
        bd.spec_kv_set_len(self.kv, B, target_len, -1)
        bd.spec_verify_forward(self.model, self.kv, B, 2, tok2, self.logits2, self.ws2)
        bd.spec_kv_set_len(self.kv, B, None, 2)
        tok = self.drafts if B == 1 else self.drafts_t  # [1, gamma] and [gamma, 1] coincide
        for i in range(g):
            if i > 0:
                bd.spec_verify_forward(self.model, self.kv, B, 1, tok[i - 1] if B > 1 else self.drafts[:, i - 1:i],
                                       self.logits1, self.ws1)
                bd.spec_kv_set_len(self.kv, B, None, 1)
                logits, ld, off = self.logits1, V, 0
            else:
                logits, ld, off = self.logits2, 2 * V, V  # the last committed token's row of each sequence
            bd.spec_draft_sample(logits, ld, B, V, self.T, u_draft[i], self.q, g * V, tok, 1 if B > 1 else g,
                                 self.sws, logits_off=off, q_off=i * V, tokens_off=i * B if B > 1 else i)
        if B > 1:
            self.drafts.copy_(self.drafts_t.t())
        return self.drafts, self.q, None


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
        # strict hit counts over the unfinished sequences' rounds
        self.hit_rounds = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.found_tokens = torch.zeros(B, dtype=torch.int32, device="cuda")

    def bind(self, committed, out, out_len, cap: int, n_stop: int = 0):
        """Set the context: committed [B] lists (the prefix rows) and the
        device buffers the rounds append to; rounds of sequences that hold
        n_stop tokens already are not counted in the hit statistics."""
        P = max(len(c) for c in committed)
        rows = np.zeros((self.B, P), dtype=np.int32)
        for b, c in enumerate(committed):
            rows[b, :len(c)] = c
        self.prefix = _dev_i32(rows)
        self.prefix_len = _dev_i32([len(c) for c in committed])
        self.P, self.out, self.out_len, self.cap, self.n_stop = P, out, out_len, cap, n_stop
        if out_len is not None:
            self.hit_rounds.zero_()
            self.found_tokens.zero_()

    def propose(self):
        bd.spec_ngram_propose(self.B, self.n, self.n_max, self.gamma, self.prefix, self.prefix_len, self.P, self.out,
                              self.out_len, self.cap, self.fill_off, self.drafts, self.n_draft, self.n_found)
        # statistics only (not part of the proposal): rounds whose lookup found
        # at least one token, and the tokens it found
        active = (self.out_len < self.n_stop).int() if (self.n_stop > 0 and self.out_len is not None) else 1
        self.hit_rounds += (self.n_found > 0).int() * active
        self.found_tokens += self.n_found * active
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
                # eager: the proposer's prefix rows are the whole committed context
                self.drafter.bind(self.committed, None, None, 0)
                drafts, nd = self.drafter.propose()
                drafts = drafts[:, :g].contiguous()
        self.last_round = (drafts, q, nd)  # this round's draft inputs, for inspection
        bd.spec_decode_step(self.target, self.kv, B, g, self.T, self.last, drafts, nd, q, u_acc if g else None,
                            u_res, self.n, self.emitted, logits_out, self.ws)
        n = self.n.cpu().numpy()
        em = self.emitted.cpu().numpy()
        for b in range(B):
            self.committed[b] += [int(t) for t in em[b, :n[b] + 1]]
        return n, em

    def generate(self, n_new: int, preload_uniforms: bool = True) -> dict:
        """Rounds until every sequence has n_new new tokens (then truncated).
        Acceptance figures count each sequence's rounds until it had n_new."""
        B, g = self.B, self.gamma
        max_rounds = n_new + 1
        pool = [self._uniforms(r) for r in range(max_rounds)] if preload_uniforms else None
        torch.cuda.synchronize()
        per_seq = [[] for _ in range(B)]
        rounds, t0 = 0, time.perf_counter()
        round_ms = []
        while min(len(c) for c in self.committed) - self.prompt_len < n_new:
            done = [len(c) - self.prompt_len >= n_new for c in self.committed]
            t1 = time.perf_counter()
            n, _ = self.round(rounds, pool[rounds] if pool else None)
            round_ms.append((time.perf_counter() - t1) * 1e3)
            for b in range(B):
                if not done[b]:
                    per_seq[b].append(int(n[b]))
            rounds += 1
        wall = time.perf_counter() - t0
        tokens = [c[self.prompt_len:self.prompt_len + n_new] for c in self.committed]
        stats = acceptance_stats(per_seq, g)
        res = {"tokens": tokens, "rounds": rounds, "wall_s": wall, "tok_s": B * n_new / wall,
               "round_ms_p50": float(np.percentile(round_ms, 50)), "round_ms_p99": float(np.percentile(round_ms, 99)),
               **stats}
        if "mean_acceptance_length" not in res:
            res["mean_acceptance_length"] = 1.0
            res["acceptance_rate"] = 0.0
        return res

    def generate_graph(self, n_new: int, check=None, logits_out=None) -> dict:
        """The rounds of generate(), with the same uniforms, run as replays of
        one captured HIP graph per round: the drafter's passes, the verify
        step and the round bookkeeping (spec_commit_round) all stay on the
        device.  Per round the host only copies that round's uniforms into the
        graph's buffers; it reads the output counts once per batch of rounds,
        each batch no longer than the fewest rounds that could finish.  A
        sequence that has its n_new tokens is frozen by spec_commit_round (its
        later rounds are discarded and its KV length restored), so the cache
        never grows past prompt + n_new + 2 gamma positions.

        ``check(r, info)``, when given, runs after every round (one replay per
        host synchronisation) with that round's inputs and outputs, for
        checking graph-replayed rounds against a reference; ``logits_out``
        [B, gamma+1, V] then receives the verify logits."""
        B, g = self.B, self.gamma
        if g > 0 and not isinstance(self.drafter, (ModelDrafter, DeviceNgramDrafter)):
            raise ValueError("graph rounds need a device drafter (ModelDrafter, DeviceNgramDrafter) or gamma = 0")
        if max(len(c) for c in self.committed) - 1 + n_new + 2 * g + 1 > self.kv.max_ctx:
            raise ValueError("KV cache too short: needs prompt + n_new + 2 gamma positions")
        cap = n_new + g + 1
        dev = "cuda"
        tok2 = _dev_i32([[c[-2], c[-1]] for c in self.committed])
        last = _dev_i32([c[-1] for c in self.committed])
        out = torch.zeros((B, cap), dtype=torch.int32, device=dev)
        out_len = torch.zeros(B, dtype=torch.int32, device=dev)
        max_rounds = n_new + 1
        n_rounds = torch.zeros(B, dtype=torch.int32, device=dev)
        n_log = torch.full((B, max_rounds), -1, dtype=torch.int32, device=dev)
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
            self.drafter.bind(self.committed, out, out_len, cap, n_new)
        drafts = q = nd = None

        def body():
            nonlocal drafts, q, nd
            if g and ngram:
                drafts, nd = self.drafter.propose()
            elif g:
                drafts, q, _ = self.drafter.draft(tok2, self.kv.len, u_draft)
            bd.spec_decode_step(self.target, self.kv, B, g, self.T, last, drafts, nd, q, u_acc, u_res, self.n,
                                self.emitted, logits_out, self.ws)
            bd.spec_commit_round(B, g, self.n, self.emitted, tok2, last, out, out_len, cap, n_new, self.kv.len,
                                 n_rounds, n_log, max_rounds)

        host_ctx = [list(c) for c in self.committed] if check else None

        def after_round(r):
            torch.cuda.synchronize()
            ol = out_len.cpu().numpy()
            toks = out.cpu().numpy()
            ctx_before = [list(c) for c in host_ctx]
            for b in range(B):
                host_ctx[b] = self.committed[b] + list(map(int, toks[b, :min(int(ol[b]), cap)]))
            u = {"u_acc": ua_all[r].cpu().numpy() if g else np.zeros((B, 0), np.float32),
                 "u_res": ur_all[r].cpu().numpy(),
                 "u_draft": ud_all[r].cpu().numpy().T if g else np.zeros((B, 0), np.float32)}
            check(r, {"context": ctx_before, "drafts": None if drafts is None else drafts[:, :g].cpu().numpy(),
                      "q": None if q is None else q.cpu().numpy(), "n_draft": None if nd is None else nd.cpu().numpy(),
                      "u": u, "n": self.n.cpu().numpy(), "emitted": self.emitted.cpu().numpy(),
                      "logits": None if logits_out is None else logits_out.cpu().numpy(),
                      "kv_len": self.kv.len.cpu().numpy(), "out_len": ol})

        # Round 0 runs eagerly (it also performs every kernel's one-time
        # set-up) and is timed; the capture that follows records the round
        # without running it and is not timed, as a server captures once.
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        load_uniforms(0)
        body()
        torch.cuda.synchronize()
        wall0 = time.perf_counter() - t0
        if check:
            after_round(0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            body()
        torch.cuda.synchronize()
        events = [torch.cuda.Event(enable_timing=True)]
        events[0].record()
        t0 = time.perf_counter()
        rounds = 1
        while rounds < max_rounds:
            remaining = n_new - int(out_len.min().item())
            if remaining <= 0:
                break
            batch = 1 if check else max(1, -(-remaining // (g + 1)))
            for _ in range(min(batch, max_rounds - rounds)):
                load_uniforms(rounds)
                graph.replay()
                ev = torch.cuda.Event(enable_timing=True)
                ev.record()
                events.append(ev)
                if check:
                    after_round(rounds)
                rounds += 1
        torch.cuda.synchronize()
        wall = wall0 + time.perf_counter() - t0
        total = out_len.cpu().numpy()
        if int(total.min()) < n_new:
            raise RuntimeError("generation did not finish within n_new + 1 rounds")
        if int(self.kv.len.max().item()) + g + 1 > self.kv.max_ctx:
            raise RuntimeError("KV length passed max_ctx")
        toks = out.cpu().numpy()
        tokens = [list(map(int, toks[b, :n_new])) for b in range(B)]
        for b in range(B):
            self.committed[b] += list(map(int, toks[b, :min(int(total[b]), cap)]))
        nr = n_rounds.cpu().numpy()
        logs = n_log.cpu().numpy()
        stats = acceptance_stats([logs[b, :nr[b]] for b in range(B)], g)
        round_ms = [events[i].elapsed_time(events[i + 1]) for i in range(len(events) - 1)] if check is None else []
        res = {"tokens": tokens, "rounds": rounds, "wall_s": wall, "tok_s": B * n_new / wall,
               "sequence_rounds": nr.tolist(), **stats}
        if "mean_acceptance_length" not in res:
            res["mean_acceptance_length"] = 1.0
            res["acceptance_rate"] = 0.0
        if round_ms:
            res["round_ms_p50"] = float(np.percentile(round_ms, 50))
            res["round_ms_p99"] = float(np.percentile(round_ms, 99))
        if ngram:
            hits = int(self.drafter.hit_rounds.sum().item())
            res["ngram_hit_rate"] = hits / max(int(nr.sum()), 1)
            res["ngram_found_tokens_per_round"] = int(self.drafter.found_tokens.sum().item()) / max(int(nr.sum()), 1)
        return res
