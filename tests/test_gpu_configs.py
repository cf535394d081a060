"""End-to-end parity on the five workload configurations: whole speculative
generations on the GPU, replayed round by round by the oracle, teacher-forced
(the oracle starts every round from the GPU's committed tokens and gets the
GPU's drafts, draft rows and uniforms).

Per round:
* verify logits within 1e-4 (fp32 models) / 2e-2 (bf16 models) of the
  oracle's own forward pass, probabilities within 1e-5.  At the 8B shape
  every step of every layer is held to the bar on the inputs the kernels had
  (tests/_layerwise.py: at d_model 4096 the bf16 rounding points put two
  faithful implementations 0.01-0.03 apart after a single layer, so whole
  passes are not comparable at 2e-2), and the logits and probabilities are
  the oracle's final RMSNorm, LM head and softmax on the GPU's last residual
  rows;
* n and emitted bit-exact against the oracle's rule run on the GPU's own p
  and q rows;
* against the oracle's own p: identical, except
  - accept decisions with u within 1e-4 of the oracle's threshold
    min(1, p/q) ("band"), or between the oracle's and the GPU's thresholds
    ("moved": the two p rows differ within the tolerances), counted per class;
  - draws whose CDF boundary moved: u lies between the two rows' normalised
    cumulative weights at the first index where the two draws part (asserted
    for every such draw, then counted).  With near-uniform rows of
    32000-151936 entries, bf16 noise moves boundaries often;
* model drafters: each drafted token equals the oracle's draw on the GPU's q
  row, and the q rows match the oracle's draft model within 1e-5 up to the
  first draw that differs.

Sizes: configs 1 and 2 run their full generations, both eagerly and as
graph-replayed rounds; the 8B config runs rounds at the workload's 256-token
prompt and near its 516-position end; the batch sweep and the n-gram config
check a seeded subset of the sequences of every batch (all when B <= 8).
"""
import numpy as np
import pytest
import torch

from draft_then_verify_amd import binding as bd
from draft_then_verify_amd.runner import DeviceNgramDrafter, ModelDrafter, SpecDecoder
from oracle import model as OM
from oracle import ngram as NG
from oracle import rounds as R
from oracle import sampler as S
from synth import SHAPES, make_markov_table, make_prompt, make_weights, markov_prompt, round_uniforms
from tests._gpu import f32, gpu_softmax, i32, to_dev
from tests._layerwise import check_passes, record_pass

pytestmark = pytest.mark.gpu


def _sub(w: dict, layers: int) -> dict:
    """The self-speculative draft's weights: the first layers plus the shared
    embedding, final norm and head."""
    out = {}
    for k, v in w.items():
        out[k] = v[:layers] if k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd") else v
    return out


def assert_cdf_shift(r_g, r_o, u, t_g, t_o):
    """Two draws with the same uniform u from two rows part only where the
    rows' normalised cumulative weights straddle u: at the first index where
    the draws part, one row's cumulative weight exceeds u and the other's
    does not.  Anything else (a wrong row, a wrong uniform, a broken scan)
    fails here."""
    wg = S.fixed_point_weights(r_g).astype(np.float64)
    wo = S.fixed_point_weights(r_o).astype(np.float64)
    v = min(t_g, t_o)
    cg, co = wg[:v + 1].sum() / wg.sum(), wo[:v + 1].sum() / wo.sum()
    assert min(cg, co) - 1e-9 <= u <= max(cg, co) + 1e-9, \
        f"draw {t_g} vs {t_o}: u={u} outside the CDF shift [{min(cg, co)}, {max(cg, co)}]"


class Decisions:
    """Counts of the decisions that may differ from the oracle's own p, each
    checked to be explained before it is counted."""

    def __init__(self):
        self.band = 0
        self.moved = 0
        self.draws = 0
        self.rounds = 0

    def report(self, what):
        print(f"[{what}] {self.rounds} rounds checked; accept decisions that flipped with u within 1e-4 of the "
              f"threshold: {self.band}; between the oracle's and the GPU's thresholds: {self.moved}; draws whose "
              f"CDF boundary moved: {self.draws}", flush=True)

    @property
    def flips(self):
        return self.band + self.moved

    def compare(self, p_o, p_g, q, drafts, nd, u_acc, u_res, n_g, em_g):
        """p_o: the oracle's p rows, p_g: the GPU's (rows of the same
        sequences); integer outputs of the GPU for those sequences."""
        Bs, g1, V = p_g.shape
        g = g1 - 1
        drafts = np.asarray(drafts, np.int64).reshape(Bs, g)
        n_o, em_o = S.reject_sample(p_o.astype(np.float32), q, drafts, nd, u_acc, u_res)
        band = np.zeros(Bs, bool)
        moved = np.zeros(Bs, bool)
        if g > 0:
            qx = np.ones((Bs, g)) if q is None else np.take_along_axis(q, drafts[:, :, None], 2)[..., 0]
            px = np.take_along_axis(p_o[:, :g], drafts[:, :, None], 2)[..., 0]
            pg = np.take_along_axis(p_g[:, :g], drafts[:, :, None], 2)[..., 0]
            th_o = np.minimum(1.0, px / np.maximum(qx, 1e-30))
            th_g = np.minimum(1.0, pg / np.maximum(qx, 1e-30))
            band = (np.abs(u_acc - th_o) < 1e-4).any(axis=1)
            moved = ((u_acc - th_o) * (u_acc - th_g) <= 0).any(axis=1)
        same_n = n_o == n_g
        assert (same_n | band | moved).all(), "an accept decision flipped without a reason"
        self.band += int((~same_n & band).sum())
        self.moved += int((~same_n & ~band & moved).sum())
        # draws: where n agrees and t differs, u must lie between the two rows'
        # normalised cumulative weights at the first index where the draws part
        ndv = np.full(Bs, g) if nd is None else np.clip(np.asarray(nd), 0, g)
        r_o = S.corrected_rows(p_o.astype(np.float32), q, drafts, n_g, ndv)
        r_g = S.corrected_rows(p_g.astype(np.float32), q, drafts, n_g, ndv)
        for j in np.nonzero(same_n)[0]:
            t_g, t_o = int(em_g[j, n_g[j]]), int(em_o[j, n_g[j]])
            if t_g != t_o:
                assert_cdf_shift(r_g[j], r_o[j], float(u_res[j]), t_g, t_o)
                self.draws += 1
        self.rounds += 1


class Replay:
    """The oracle's side of a teacher-forced generation for a subset of the
    GPU's sequences (models of at most 8 layers: whole passes against the bar)."""

    def __init__(self, shape, w_host, prompt, rows, max_ctx, draft_shape=None, w_draft=None, precast=True):
        self.rows = np.asarray(rows)
        self.tgt = OM.Decoder(shape, w_host, precast=precast)
        self.ct = self.tgt.new_cache(len(rows), max_ctx)
        R.prefill(self.tgt, self.ct, prompt[self.rows])
        self.dft = None
        if draft_shape is not None:
            self.dft = OM.Decoder(draft_shape, w_draft, precast=precast)
            self.cd = self.dft.new_cache(len(rows), max_ctx)
            R.prefill(self.dft, self.cd, prompt[self.rows])
        self.tol = 1e-4 if shape.dtype == "f32" else 2e-2
        self.dec = Decisions()

    def report(self, what):
        self.dec.report(what)

    def check_draft(self, committed, drafts_g, q_g, u_draft):
        """q rows of the GPU drafter against the oracle draft model, teacher-forced."""
        r = self.rows
        prev = np.array([committed[b][-2] for b in r])
        last = np.array([committed[b][-1] for b in r])
        tl = self.ct.length.copy()
        g = drafts_g.shape[1]
        d_o, q_o = R.draft_round(self.dft, self.cd, prev, last, tl, g, u_draft[r])
        for j, b in enumerate(r):
            for i in range(g):
                # the GPU's draw is the oracle's rule on the GPU's own row
                assert S.sample(q_g[b, i][None], u_draft[b, i][None])[0] == drafts_g[b, i]
                err = np.abs(q_g[b, i] - q_o[j, i]).max()
                assert err < 1e-5, f"round {self.dec.rounds} seq {b} draft step {i}: q differs by {err:.3g}"
                if d_o[j, i] != drafts_g[b, i]:
                    assert_cdf_shift(q_g[b, i], q_o[j, i], float(u_draft[b, i]), int(drafts_g[b, i]), int(d_o[j, i]))
                    self.dec.draws += 1
                    break
        # teacher forcing: the oracle draft cache holds the GPU's drafted tokens
        self.cd.length = tl - 1
        self.dft.forward(self.cd, np.concatenate([prev[:, None], last[:, None], drafts_g[r][:, :g - 1]], axis=1),
                         logits=False)

    def check_round(self, last, drafts, q, nd, u, logits_g, n_g, em_g):
        r = self.rows
        len0 = self.ct.length.copy()
        qs = None if q is None else q[r]
        nds = None if nd is None else nd[r]
        out = R.verify_round(self.tgt, self.ct, last[r], drafts[r], qs, nds, u["u_acc"][r], u["u_res"][r])
        dev = np.abs(logits_g[r] - out["logits"])
        assert dev.max() < self.tol, f"logits differ by {dev.max():.3g}"
        V = logits_g.shape[-1]
        p_g = gpu_softmax(torch.as_tensor(logits_g[r]).cuda(), V).cpu().numpy()
        assert np.abs(p_g - out["p"]).max() < 1e-5
        n_own, em_own = S.reject_sample(p_g, qs, drafts[r], nds, u["u_acc"][r], u["u_res"][r])
        assert np.array_equal(n_own, n_g[r]) and np.array_equal(em_own, em_g[r])
        self.dec.compare(out["p"], p_g, qs, drafts[r], nds, u["u_acc"][r], u["u_res"][r], n_g[r], em_g[r])
        # teacher forcing: follow the GPU's commit
        self.ct.length = len0 + n_g[r] + 1


def _run(dec, replay, n_rounds, u_seed, check_draft=False, stop_at=None):
    B, g, V = dec.B, dec.gamma, dec.V
    logits = torch.empty((B, g + 1, V), dtype=torch.float32, device="cuda")
    r = 0
    while r < n_rounds:
        if stop_at is not None and min(len(c) for c in dec.committed) - dec.prompt_len >= stop_at:
            break
        u = round_uniforms(u_seed, r, B, g)
        uni = (torch.as_tensor(u["u_acc"]).cuda(), torch.as_tensor(u["u_res"]).cuda(),
               torch.as_tensor(np.ascontiguousarray(u["u_draft"].T)).cuda())
        committed_before = [list(c) for c in dec.committed]
        last = np.array([c[-1] for c in committed_before])
        n_g, em_g = dec.round(r, uni, logits_out=logits)
        drafts, q, nd = dec.last_round
        drafts = drafts.cpu().numpy().astype(np.int64)
        q = None if q is None else q.cpu().numpy()
        nd = None if nd is None else nd.cpu().numpy()
        if check_draft:
            replay.check_draft(committed_before, drafts, q, u["u_draft"])
        replay.check_round(last, drafts, q, nd, u, logits.cpu().numpy(), n_g, em_g)
        # round invariants
        assert ((n_g >= 0) & (n_g <= g)).all()
        for b in range(B):
            assert (em_g[b, n_g[b] + 1:] == -1).all() and (em_g[b, :n_g[b]] == drafts[b, :n_g[b]]).all()
        r += 1
    return r


def _self_spec(shape_name, seed, P, N, draft_layers, g=4):
    sh = SHAPES[shape_name]
    w = make_weights(sh, seed=seed)
    dsh = sh.with_(n_layers=draft_layers)
    max_ctx = P + N + 2 * g + 4
    prompt = make_prompt(1, P, sh.vocab, seed=seed)
    target = bd.SpecModel(sh, to_dev(w))
    draft = bd.SpecModel(dsh, to_dev(_sub(w, draft_layers)))
    dec = SpecDecoder(target, 1, g, max_ctx, drafter=ModelDrafter(draft, 1, g, max_ctx), seed=seed)
    dec.prefill(prompt)
    rep = Replay(sh, w, prompt, [0], max_ctx, dsh, _sub(w, draft_layers))
    return sh, dec, rep


def test_config1_tiny_full_generation():
    """Tiny fp32 target, self-speculative 1-layer draft, B=1, gamma=4, 64-token
    prompt, 32 new tokens: every round of the whole generation."""
    P, N = 64, 32
    sh, dec, rep = _self_spec("tiny", 301, P, N, 1)
    rounds = _run(dec, rep, N + 1, 301, check_draft=True, stop_at=N)
    assert len(dec.committed[0]) - P >= N
    rep.report('config 1')
    assert rep.dec.flips <= max(1, rounds // 10)


def test_config2_small_full_generation():
    """Small bf16 target (8 layers, 16/4 heads), self-speculative 2-layer draft,
    B=1, gamma=4, 512-token prompt, 256 new tokens: every round."""
    P, N = 512, 256
    sh, dec, rep = _self_spec("small", 302, P, N, 2)
    rounds = _run(dec, rep, N + 1, 302, check_draft=True, stop_at=N)
    assert len(dec.committed[0]) - P >= N
    rep.report('config 2')
    assert rep.dec.flips <= max(2, rounds // 10)


def _graph_checked(shape_name, seed, P, N, draft_layers):
    """A graph-replayed generation, every round replayed by the oracle from
    what the graph's buffers held after that round."""
    g = 4
    sh, dec, rep = _self_spec(shape_name, seed, P, N, draft_layers)
    logits = torch.empty((1, g + 1, sh.vocab), dtype=torch.float32, device="cuda")
    seen = []

    def check(r, info):
        ctx = info["context"]
        assert len(ctx[0]) - P < N  # one sequence: no round after it has its tokens
        last = np.array([c[-1] for c in ctx])
        rep.check_draft(ctx, info["drafts"], info["q"], info["u"]["u_draft"])
        rep.check_round(last, info["drafts"], info["q"], info["n_draft"], info["u"], info["logits"], info["n"],
                        info["emitted"])
        assert int(info["kv_len"][0]) == len(ctx[0]) - 1 + int(info["n"][0]) + 1
        seen.append(r)

    res = dec.generate_graph(N, check=check, logits_out=logits)
    assert seen == list(range(len(seen))) and len(seen) == res["rounds"]
    rep.report(f"graph rounds, {shape_name}")
    return res, rep


def test_config1_graph_rounds_oracle():
    """Config 1 as graph replays (drafter passes, verify step and bookkeeping
    on the device): every replayed round against the oracle."""
    res, rep = _graph_checked("tiny", 311, 64, 32, 1)
    assert rep.dec.flips <= max(1, res["rounds"] // 10)


def test_config2_graph_rounds_oracle():
    """Config 2 (512-token prompt, 256 new tokens) as graph replays: every
    replayed round against the oracle."""
    res, rep = _graph_checked("small", 312, 512, 256, 2)
    assert rep.dec.flips <= max(2, res["rounds"] // 10)


def _draft_pass(draft, kvd, tokens, m, records, name):
    logits = torch.empty((1, m, draft.shape.vocab), dtype=torch.float32, device="cuda")
    records.append(record_pass(name, draft, kvd, 1, m, i32(np.asarray(tokens).reshape(1, m)), logits))
    bd.spec_kv_set_len(kvd, 1, None, m)
    return logits[:, -1]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("P", [256, 508])
def test_config3_8b_layerwise(P):
    """The 8B-shaped target with the 0.6B-shaped drafter, B=1, gamma=4, at the
    full model shapes and the workload's context: a P-token prompt (256, and
    508 so that the verify rows attend to 508-517 keys, the end of a 256-token
    generation), then two rounds.  Every step of every layer of every verify
    and drafter pass is held to the bar on the inputs the kernels had; the
    first, a middle and the last layer of the two prefills (the matrix-core
    path) too.  The rounds are driven here through the C ABI in the order the
    generation driver uses."""
    tsh, dsh = SHAPES["qwen3_8b"], SHAPES["qwen3_0p6b"]
    g, V, seed = 4, SHAPES["qwen3_8b"].vocab, 303
    max_ctx = P + 3 * (g + 1) + 4
    wt = make_weights(tsh, seed=seed, device="cuda", norm="random")
    wd = make_weights(dsh, seed=seed + 1, device="cuda", norm="random")
    target, draft = bd.SpecModel(tsh, wt), bd.SpecModel(dsh, wd)
    kvt = bd.KVCache(tsh, tsh.n_layers, 1, max_ctx)
    kvd = bd.KVCache(dsh, dsh.n_layers, 1, max_ctx)
    prompt = make_prompt(1, P, V, seed=seed)
    trec, drec = [], []
    trec.append(record_pass("target prefill", target, kvt, 1, P - 1, i32(prompt[:, :-1]), None))
    bd.spec_kv_set_len(kvt, 1, None, P - 1)
    drec.append(record_pass("draft prefill", draft, kvd, 1, P - 1, i32(prompt[:, :-1]), None))
    bd.spec_kv_set_len(kvd, 1, None, P - 1)
    ctx = list(map(int, prompt[0]))
    sws = bd.workspace(bd.spec_sampler_workspace_bytes(g + 1, 1, V))
    wsd = bd.workspace(target.workspace_bytes(1, g + 1, max_ctx))
    n_d = torch.empty(1, dtype=torch.int32, device="cuda")
    em_d = torch.empty((1, g + 1), dtype=torch.int32, device="cuda")
    x_d = torch.empty((1, 1), dtype=torch.int32, device="cuda")
    rounds = []
    for r in range(2):
        u = round_uniforms(seed, r, 1, g)
        # drafter: rewind to the target's length - 1, re-feed the last two
        # committed tokens, then one row per drafted token
        bd.spec_kv_set_len(kvd, 1, kvt.len, -1)
        qs, xs = [], []
        row = _draft_pass(draft, kvd, ctx[-2:], 2, drec, f"round {r} draft pass 0")
        for i in range(g):
            if i > 0:
                row = _draft_pass(draft, kvd, [xs[-1]], 1, drec, f"round {r} draft pass {i}")
            q_i = gpu_softmax(row.contiguous(), V)
            bd.spec_reject_sample(1, 0, V, q_i, None, None, None, None, f32(u["u_draft"][:, i]), n_d, x_d, sws)
            qs.append(q_i.cpu().numpy()[0])
            xs.append(int(x_d.item()))
        drafts = np.array([xs], np.int64)
        q = np.stack(qs)[None]
        # verify: the pass with its residual rows, then the decode step itself
        tokens = i32(np.array([[ctx[-1]] + xs]))
        lg_h = torch.empty((1, g + 1, V), dtype=torch.float32, device="cuda")
        trec.append(record_pass(f"round {r} verify", target, kvt, 1, g + 1, tokens, lg_h))
        lg = torch.empty_like(lg_h)
        bd.spec_decode_step(target, kvt, 1, g, 1.0, i32([ctx[-1]]), i32(drafts), None, f32(q), f32(u["u_acc"]),
                            f32(u["u_res"]), n_d, em_d, lg, wsd)
        torch.cuda.synchronize()
        assert torch.equal(lg, lg_h), "the decode step's pass differs from the recorded pass"
        n, em = n_d.cpu().numpy(), em_d.cpu().numpy()
        rounds.append((drafts, q, u, n, em))
        ctx += [int(t) for t in em[0, :n[0] + 1]]
        assert int(kvt.len.item()) == len(ctx) - 1
    # prefills: the first, a middle and the last layer; passes of rounds: all layers
    prefill_layers = lambda L: (lambda rec: {0, L // 2, L - 1} if "prefill" in rec.name else range(L))
    lo_t = check_passes(tsh, wt, trec, 2e-2, prefill_layers(tsh.n_layers))
    lo_d = check_passes(dsh, wd, drec, 2e-2, prefill_layers(dsh.n_layers))
    dec = Decisions()
    for r, (drafts, q, u, n, em) in enumerate(rounds):
        # drafter: the GPU's draws are the oracle's rule on the GPU's rows, and
        # the rows are the oracle's softmax of its teacher-forced logits
        for i in range(g):
            assert S.sample(q[0, i][None], u["u_draft"][:, i])[0] == drafts[0, i]
            q_o = S.softmax(lo_d[f"round {r} draft pass {i}"][0, -1])
            assert np.abs(q[0, i] - q_o).max() < 1e-5
        lg = trec[1 + r].logits
        p_g = gpu_softmax(torch.as_tensor(lg).cuda(), V).cpu().numpy()
        p_o = S.softmax(lo_t[f"round {r} verify"])
        assert np.abs(p_g - p_o).max() < 1e-5
        n_own, em_own = S.reject_sample(p_g, q, drafts, None, u["u_acc"], u["u_res"])
        assert np.array_equal(n_own, n) and np.array_equal(em_own, em)
        dec.compare(p_o, p_g, q, drafts, None, u["u_acc"], u["u_res"], n, em)
    dec.report(f"config 3, prompt {P}")
    assert dec.flips <= 1


@pytest.mark.parametrize("B", [1, 8, 64, 256])
def test_config4_batch_sweep_round(B):
    """Config-2 shapes at B sequences (verify M = 5B rows), 2-layer
    self-speculative draft: two rounds; the oracle replays every sequence for
    B <= 8, 8 seeded sequences otherwise.  Prompts are 256 tokens (the
    prefill of B x 255 rows runs on the matrix cores)."""
    sh = SHAPES["small"]
    w = make_weights(sh, seed=304)
    dsh = sh.with_(n_layers=2)
    P, g = 256, 4
    max_ctx = P + 2 * (g + 1) + 4
    prompt = make_prompt(B, P, sh.vocab, seed=304 + B)
    target = bd.SpecModel(sh, to_dev(w))
    draft = bd.SpecModel(dsh, to_dev(_sub(w, 2)))
    dec = SpecDecoder(target, B, g, max_ctx, drafter=ModelDrafter(draft, B, g, max_ctx), seed=304)
    dec.prefill(prompt)
    rows = np.arange(B) if B <= 8 else np.sort(np.random.default_rng(B).choice(B, 8, replace=False))
    rep = Replay(sh, w, prompt, rows, max_ctx, dsh, _sub(w, 2))
    rounds = _run(dec, rep, 2, 304 + B, check_draft=True)
    rep.report(f'{__name__}')
    assert rounds == 2 and rep.dec.flips <= 1


@pytest.mark.parametrize("B", [1, 64])
def test_config5_ngram_long_draft(B):
    """n-gram drafter (trigram prompt lookup on the device, one-hot q) on the
    config-2 body with V = 151936, gamma = 10, order-2 Markov prompts: two
    rounds; the oracle replays every sequence for B = 1, 8 seeded sequences
    of 64, and its own lookup must propose what the device proposed.  Misses
    are filled with the gamma tokens after a seeded prompt offset so every
    round verifies B x 11 rows.  Prompts are 2048 tokens (the prefill of
    64 x 2047 rows runs on the matrix cores)."""
    sh = SHAPES["small_v151936"]
    w = make_weights(sh, seed=305)
    P, g = 2048, 10
    max_ctx = P + 2 * (g + 1) + 4
    table = make_markov_table(seed=305)
    prompt = markov_prompt(B, P, table, seed=305 + B).astype(np.int64)
    offs = np.random.default_rng(305).integers(0, P - g - 1, size=B)
    target = bd.SpecModel(sh, to_dev(w))
    drafter = DeviceNgramDrafter(B, g, n=3, fill_off=offs)
    dec = SpecDecoder(target, B, g, max_ctx, drafter=drafter, seed=305)
    dec.prefill(prompt)
    rows = np.arange(B) if B <= 8 else np.sort(np.random.default_rng(B).choice(B, 8, replace=False))
    rep = Replay(sh, w, prompt, rows, max_ctx)
    contexts = [[list(c) for c in dec.committed]]
    orig_round = dec.round

    def round_and_keep(r, uniforms=None, logits_out=None):
        contexts.append(None)
        out = orig_round(r, uniforms, logits_out)
        contexts[-1] = [list(c) for c in dec.committed]
        return out

    dec.round = round_and_keep
    rounds = _run(dec, rep, 2, 305 + B)
    # the device lookup proposed what the oracle's lookup (with the same fill) proposes
    drafts, _, nd = dec.last_round
    ctx = contexts[-2]
    for b in rows:
        prop = NG.ngram_propose(ctx[b], 3, g)
        prop = prop + [int(t) for t in prompt[b, offs[b]:offs[b] + g - len(prop)]]
        assert drafts[b, :g].cpu().tolist() == prop
    rep.report(f'{__name__}')
    assert rounds == 2 and rep.dec.flips <= 1
