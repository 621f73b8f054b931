"""The successor-planted stack of the synthetic inputs: a stand-in for a trained model that has
learned a history's successor statistics, used by the prompt-lookup loop (random-init weights
follow no text, so the n-gram drafter would never find what they say).  Checked on the host:
the successor map against brute-force counting, the layer scaling against exact float
arithmetic, and, through the oracle, that the stack's greedy choice after a token is that
token's successor, whatever precedes it."""
import collections

import numpy as np

import oracle
import synth

S = synth.TINY


def test_history_successors_match_brute_force_counts():
    rng = np.random.default_rng(3)
    vocab = 40
    hist = rng.integers(0, 12, size=300).astype(np.int32)   # ids 12..39 never occur
    hist[::7] = 5                                            # many ties and repeats
    succ = synth.history_successors(hist, vocab, 17)
    follow = collections.defaultdict(collections.Counter)
    for a, b in zip(hist[:-1].tolist(), hist[1:].tolist()):
        follow[a][b] += 1
    for a, cnt in follow.items():
        best = max(cnt.values())
        assert succ[a] == min(b for b, c in cnt.items() if c == best), a
    again = synth.history_successors(hist, vocab, 17)
    assert (succ == again).all() and succ.min() >= 0 and succ.max() < vocab
    assert set(range(12, vocab)).isdisjoint(follow)          # those got the seeded ids


def test_successor_stack_scales_layers_exactly_and_builds_the_head():
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    succ = synth.history_successors(synth.lookup_history(S.vocab, 400, 7), S.vocab, 3)
    wp = synth.successor_stack(w, succ, shift=8)

    def f32(u):
        return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    for name in ("l0.wq", "l1.wd", "l0.bk"):
        assert np.array_equal(f32(wp[name]), f32(w[name]) * 2.0 ** -8), name
    for name in ("embed", "l0.ln1", "final_norm"):
        assert wp[name] is w[name]
    e = f32(w["embed"])
    head = f32(wp["lm_head"])
    for v in (int(succ[0]), int(succ[123]), 7, 4000):
        pre = np.flatnonzero(succ == v)
        want = e[pre].sum(axis=0) if len(pre) else np.zeros(S.hidden)
        assert np.allclose(head[v], want, rtol=2 ** -7, atol=1e-6), v


def test_successor_stack_greedy_choice_is_the_successor():
    """Prompts ending in a token t, of a few lengths: the oracle's greedy next token is succ[t],
    by a wide gap."""
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    hist = synth.lookup_history(S.vocab, 400, 7)
    succ = synth.history_successors(hist, S.vocab, 3)
    model = oracle.Model(S, synth.successor_stack(w, succ))
    rng = np.random.default_rng(11)
    for n in (1, 5, 40):
        for _ in range(3):
            prompt = rng.integers(0, S.vocab, size=n).astype(np.int32)
            c = oracle.KVCache(S, 64)
            z = oracle.prefill(model, c, prompt)
            assert c.next_token == succ[prompt[-1]], (n, prompt[-1])
            assert oracle.top_gap(z[-1:])[0].item() > 1.0


def test_perturb_successors_changes_the_stated_fraction():
    """The drafter's successor map of the device round: every id keeps its successor except a
    seeded fraction, which get uniform ids; the same seed gives the same map."""
    succ = synth.history_successors(synth.lookup_history(5000, 20000, 4), 5000, 9)
    out = synth.perturb_successors(succ, 0.22, 31)
    assert out.dtype == np.int32 and out.shape == succ.shape
    assert out.min() >= 0 and out.max() < len(succ)
    changed = np.mean(out != succ)
    assert 0.19 < changed < 0.23, changed          # 0.22 less the 1/5000 that redraw the same id
    assert np.array_equal(out, synth.perturb_successors(succ, 0.22, 31))
    assert not np.array_equal(out, synth.perturb_successors(succ, 0.22, 32))
    assert np.array_equal(synth.perturb_successors(succ, 0.0, 31), succ)
