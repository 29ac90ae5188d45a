"""Checks that pin the fp64 oracle to things other than itself.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
``AssertionError`` when the oracle disagrees with what the pages, the
mathematics or an independent library routine fix:

* special cases that reduce to a library routine (bag size 1 is
  ``index_select``; bags match ``torch.nn.functional.embedding_bag`` in fp64;
  Linear matches ``torch.addmm``; the interaction matches
  ``bmm(S, S^T)[:, li, lj]`` with ``torch.tril_indices``);
* integer-exact brute force (integer tables / vectors summed with int64);
* closed forms and counts (pair count C(F, 2), the closed-form pair index is a
  bijection in nested-loop order for F <= 64, sigmoid(0) = 0.5);
* invariants (the Gram matrix is symmetric, Z is its strict lower triangle);
* worked examples under ``tests/golden`` (the pair order and shape rules the
  pages print, and a hand-derived forward with exact dyadic values);
* an independent fp64 PyTorch eager DLRMv1 built from ``nn.EmbeddingBag``,
  ``bmm`` and ``nn.Linear``.

The battery is run against the real oracle (tests/test_oracle_pins.py) and
against copies with planted mistakes (tests/test_oracle_mutants.py), each of
which must fail at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

import dlrm_inputs as di

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# --- embedding bag --------------------------------------------------------------


def pin_embbag_bag1_is_index_select(o):
    """Bag size 1 is a plain row lookup (LessonsLearned 'EmbeddingBag translator gap', K = 1)."""
    r = _rng(1)
    T, B, D = 3, 37, 16
    tables = [r.standard_normal((50 + 7 * t, D)).astype(np.float32) for t in range(T)]
    idx = [r.integers(0, tb.shape[0], B).astype(np.int64) for tb in tables]
    off = [np.arange(B, dtype=np.int64) for _ in range(T)]
    E = o.embbag_sum(tables, idx, off)
    for t in range(T):
        ref = torch.index_select(torch.from_numpy(tables[t]), 0, torch.from_numpy(idx[t])).double().numpy()
        assert np.array_equal(E[:, t, :], ref), "bag-1 embedding bag differs from index_select"


def pin_embbag_matches_torch_embedding_bag(o):
    """Ragged bags with empty ones, against PyTorch's embedding_bag(mode='sum') in fp64."""
    T, B, D = 4, 29, 8
    r = _rng(2)
    tables, idx, off = [], [], []
    for t in range(T):
        o_t, n = di.ragged_bags(B, 6, 100 + t, empty_frac=0.3)
        tables.append(r.standard_normal((40, D)).astype(np.float32))
        idx.append(r.integers(0, 40, n).astype(np.int64))
        off.append(o_t.numpy())
    E = o.embbag_sum(tables, idx, off)
    for t in range(T):
        ref = torch.nn.functional.embedding_bag(torch.from_numpy(idx[t]), torch.from_numpy(tables[t]).double(),
                                                torch.from_numpy(off[t]), mode="sum").numpy()
        np.testing.assert_allclose(E[:, t, :], ref, rtol=1e-12, atol=1e-12)


def pin_embbag_integer_tables_exact(o):
    """Integer tables in [-8, 8], bags of 20: brute-force int64 sums, exact."""
    r = _rng(3)
    T, B, D, L, V = 2, 11, 12, 20, 64
    tables_i = [r.integers(-8, 9, (V, D)).astype(np.int64) for _ in range(T)]
    idx = [r.integers(0, V, B * L).astype(np.int64) for _ in range(T)]
    off = [np.arange(B, dtype=np.int64) * L for _ in range(T)]
    E = o.embbag_sum([t.astype(np.float32) for t in tables_i], idx, off)
    for t in range(T):
        for b in range(B):
            acc = np.zeros(D, np.int64)
            for k in range(b * L, (b + 1) * L):
                acc += tables_i[t][idx[t][k]]
            assert np.array_equal(E[b, t], acc.astype(np.float64)), f"bag ({b},{t}) differs"


def pin_embbag_rejects_malformed(o):
    """Out-of-range indices and decreasing offsets are reported, not computed."""
    import oracle as orc
    tab = [np.zeros((5, 4), np.float32)]
    bad_cases = [
        ([np.array([0, 5], np.int64)], [np.array([0, 1], np.int64)]),       # index == rows
        ([np.array([0, -1], np.int64)], [np.array([0, 1], np.int64)]),      # negative index
        ([np.array([0, 1], np.int64)], [np.array([1, 0], np.int64)]),       # decreasing offsets
        ([np.array([0, 1], np.int64)], [np.array([0, 3], np.int64)]),       # offset past the end
    ]
    for idx, off in bad_cases:
        try:
            o.embbag_sum(tab, idx, off)
        except orc.OracleError as e:
            assert e.code == orc.E_INDEX
        else:
            raise AssertionError("malformed bag input accepted")


def _ragged_case(seed, T=3, B=23, D=6, V=30, max_len=6, with_pad=True):
    r = _rng(seed)
    tables, idx, off = [], [], []
    for t in range(T):
        o, n = di.ragged_bags(B, max_len, seed * 10 + t, empty_frac=0.25)
        tables.append(r.standard_normal((V, D)).astype(np.float32))
        ix = r.integers(0, V, n).astype(np.int64)
        if with_pad and n:
            ix[r.random(n) < 0.2] = 3          # padding index 3 appears often
        idx.append(ix)
        off.append(o.numpy())
    return tables, idx, off


def pin_embbag_ex_matches_torch_embedding_bag(o):
    """mode sum / mean / max, per-sample weights, include_last_offset and padding_idx
    against torch.nn.functional.embedding_bag in fp64 (the general bag of the
    LessonsLearned 'EmbeddingBag translator gap' entry, whose follow-ups these are)."""
    F_ = torch.nn.functional
    for mode in ("sum", "mean", "max"):
        for last in (False, True):
            for pad in (None, 3):
                for weighted in ((False, True) if mode == "sum" else (False,)):
                    tables, idx, off = _ragged_case(11 + len(mode) + 2 * last + 3 * (pad is not None) + 5 * weighted)
                    r = _rng(99)
                    psw = [r.standard_normal(i.shape[0]).astype(np.float32) for i in idx] if weighted else None
                    offs = [np.concatenate([ob, [ix.shape[0]]]) for ob, ix in zip(off, idx)] if last else off
                    got = o.embbag_ex(tables, idx, offs, mode=mode, include_last_offset=last, padding_idx=pad,
                                      per_sample_weights=psw)
                    for t in range(len(tables)):
                        ref = F_.embedding_bag(torch.from_numpy(idx[t]), torch.from_numpy(tables[t]).double(),
                                               torch.from_numpy(offs[t]), mode=mode,
                                               per_sample_weights=(torch.from_numpy(psw[t]).double() if weighted
                                                                   else None),
                                               include_last_offset=last, padding_idx=pad).numpy()
                        np.testing.assert_allclose(got[:, t, :], ref, rtol=1e-12, atol=1e-12,
                                                   err_msg=f"{mode} last={last} pad={pad} w={weighted}")


def pin_embbag_ex_brute_force_integer(o):
    """Integer tables: max is exact, sum exact, mean = exact sum / count; brute force in int64."""
    r = _rng(12)
    T, B, D, V = 2, 17, 5, 40
    tables_i = [r.integers(-8, 9, (V, D)).astype(np.int64) for _ in range(T)]
    idx, off = [], []
    for t in range(T):
        o_, n = di.ragged_bags(B, 7, 700 + t)
        idx.append(r.integers(0, V, n).astype(np.int64))
        off.append(o_.numpy())
    tf = [t.astype(np.float32) for t in tables_i]
    for mode in ("sum", "mean", "max"):
        got = o.embbag_ex(tf, idx, off, mode=mode, padding_idx=[5, None])
        for t in range(T):
            ends = list(off[t][1:]) + [idx[t].shape[0]]
            for b in range(B):
                ks = [k for k in range(off[t][b], ends[b]) if not (t == 0 and idx[t][k] == 5)]
                rows_ = [tables_i[t][idx[t][k]] for k in ks]
                if not rows_:
                    want = np.zeros(D)
                elif mode == "sum":
                    want = np.sum(rows_, 0).astype(np.float64)
                elif mode == "mean":
                    want = np.sum(rows_, 0).astype(np.float64) / len(rows_)
                else:
                    want = np.max(rows_, 0).astype(np.float64)
                assert np.array_equal(got[b, t], want), (mode, t, b)


def pin_embbag_ex_last_offset_is_a_slice_end(o):
    """With include_last_offset the last bag is indices[off[B-1]:off[B]] (the pages'
    offsets[b]:offsets[b+1] slice); a final offset short of the index count leaves
    the trailing indices out.  Brute force with numpy slicing."""
    r = _rng(14)
    D, V, B = 3, 20, 6
    tab = r.standard_normal((V, D)).astype(np.float32)
    idx = r.integers(0, V, 15).astype(np.int64)
    off = np.array([0, 2, 2, 5, 9, 11, 12], np.int64)          # B + 1 entries, 12 < 15
    got = o.embbag_ex([tab], [idx], [off], mode="sum", include_last_offset=True)
    for b in range(B):
        want = tab[idx[off[b]:off[b + 1]]].astype(np.float64).sum(0) if off[b + 1] > off[b] else np.zeros(D)
        np.testing.assert_allclose(got[b, 0], want, rtol=1e-13, atol=1e-13)


def pin_embbag_ex_int32_equals_int64(o):
    """The same bags addressed with int32 indices and offsets give the same result."""
    tables, idx, off = _ragged_case(13, with_pad=False)
    a = o.embbag_ex(tables, idx, off, mode="mean")
    b = o.embbag_ex(tables, [i.astype(np.int32) for i in idx], [x.astype(np.int32) for x in off], mode="mean")
    assert np.array_equal(a, b)
    # and sum mode without options is the plain bag sum
    assert np.array_equal(o.embbag_ex(tables, idx, off), o.embbag_sum(tables, idx, off))


# --- interaction --------------------------------------------------------------


def _tril(F):
    li, lj = torch.tril_indices(F, F, offset=-1)
    return li, lj


def pin_interact_matches_bmm_tril(o):
    """Z = bmm(S, S^T)[:, li, lj] (vanilla-pytorch commit, Translator: index.Tensor peephole)."""
    r = _rng(4)
    for T, D in ((1, 3), (3, 16), (8, 5), (32, 64)):
        B = 5
        x = r.standard_normal((B, D))
        E = r.standard_normal((B, T, D))
        Z = o.interact(x, E)
        S = torch.cat([torch.from_numpy(x)[:, None, :], torch.from_numpy(E)], 1)
        G = torch.bmm(S, S.transpose(1, 2).contiguous())
        li, lj = _tril(T + 1)
        np.testing.assert_allclose(Z, G[:, li, lj].numpy(), rtol=1e-12, atol=1e-12)


def pin_interact_integer_exact(o):
    """Integer vectors with |v| <= 16: every dot is exact; brute force in int64."""
    r = _rng(5)
    B, T, D = 4, 6, 64
    x = r.integers(-16, 17, (B, D))
    E = r.integers(-16, 17, (B, T, D))
    Z = o.interact(x.astype(np.float64), E.astype(np.float64))
    for b in range(B):
        S = [x[b]] + [E[b, t] for t in range(T)]
        ref = [int(np.dot(S[i], S[j])) for i in range(T + 1) for j in range(i)]
        assert np.array_equal(Z[b], np.array(ref, np.float64))


def pin_interact_pair_order_golden(o):
    """Pair order of the pages' worked case n_feat = 4 (golden file).

    Vector f is prime_f * e_0, so the dot of (i, j) is prime_i * prime_j and
    names its pair uniquely.
    """
    g = golden("pair_order_F4.json")
    F = g["n_feat"]
    primes = [2, 3, 5, 7]
    D = 3
    x = np.zeros((1, D))
    x[0, 0] = primes[0]
    E = np.zeros((1, F - 1, D))
    for t in range(F - 1):
        E[0, t, 0] = primes[t + 1]
    Z = o.interact(x, E)[0]
    assert Z.shape[0] == g["n_pairs"]
    for p, (i, j) in enumerate(g["pairs_in_order"]):
        assert Z[p] == primes[i] * primes[j], f"pair {p} is not ({i},{j})"


def pin_gram_symmetric_and_consistent(o):
    r = _rng(6)
    B, T, D = 3, 9, 7
    x = r.standard_normal((B, D))
    E = r.standard_normal((B, T, D))
    G = o.gram(x, E)
    assert np.array_equal(G, np.transpose(G, (0, 2, 1))), "Gram matrix not symmetric"
    Z = o.interact(x, E)
    li, lj = _tril(T + 1)
    assert np.array_equal(Z, G[:, li.numpy(), lj.numpy()]), "Z is not the strict lower triangle of G"
    # diagonal entries are squared norms
    n2 = np.concatenate([(x * x).sum(1)[:, None], (E * E).sum(2)], 1)
    np.testing.assert_allclose(np.diagonal(G, axis1=1, axis2=2), n2, rtol=1e-13)


def pin_pair_count(o):
    """P = F(F-1)/2 = C(F, 2) (dlrm_megakernel.rs n_pairs); the interaction emits P values."""
    for F in range(1, 65):
        assert o.n_pairs(F) == math.comb(F, 2)
    r = _rng(7)
    for T in (1, 2, 5, 26, 32, 63):
        Z = o.interact(r.standard_normal((2, 3)), r.standard_normal((2, T, 3)))
        assert Z.shape == (2, math.comb(T + 1, 2))


def pin_pair_closed_form_bijection(o):
    """Closed form p -> (i, j) (vanilla-pytorch commit, cuda_lite kernels), brute-forced for F <= 64."""
    for F in range(2, 65):
        P = math.comb(F, 2)
        got = [o.pair_closed_form(p) for p in range(P)]
        want = [(i, j) for i in range(F) for j in range(i)]
        assert got == want, f"closed form differs from nested-loop order at F={F}"
        assert len(set(got)) == P
        assert set(got) == set((i, j) for i, j in itertools.product(range(F), range(F)) if j < i)


# --- linear layers and sigmoid ------------------------------------------------


def pin_linear_matches_addmm(o):
    """Linear = addmm(bias, x, W^T), alpha = beta = 1 (vanilla-pytorch commit, Translator)."""
    r = _rng(8)
    for (M, N, K) in ((7, 5, 3), (33, 17, 70), (4, 1, 256), (9, 64, 13)):
        x = r.standard_normal((M, K))
        W = r.standard_normal((N, K)).astype(np.float32)
        b = r.standard_normal(N).astype(np.float32)
        ref = torch.addmm(torch.from_numpy(b).double(), torch.from_numpy(x),
                          torch.from_numpy(W).double().t())
        for act, f in ((0, lambda t: t), (1, torch.relu), (2, torch.sigmoid)):
            y = o.linear(x, W, b, act)
            np.testing.assert_allclose(y, f(ref).numpy(), rtol=1e-12, atol=1e-13)
        y = o.linear(x, W, None, 0)
        np.testing.assert_allclose(y, (torch.from_numpy(x) @ torch.from_numpy(W).double().t()).numpy(),
                                   rtol=1e-12, atol=1e-13)


def pin_sigmoid_special_values(o):
    """Zero weights and bias give sigmoid(0) = 0.5 exactly; large logits saturate."""
    x = _rng(9).standard_normal((6, 8))
    W = np.zeros((1, 8), np.float32)
    assert np.all(o.linear(x, W, np.zeros(1, np.float32), 2) == 0.5)
    assert np.all(o.linear(x, W, np.full(1, 40.0, np.float32), 2) == 1.0)
    y = o.linear(x, W, np.full(1, -40.0, np.float32), 2)
    assert np.all((y > 0) & (y < 1e-17))
    y = o.linear(x, W, np.full(1, 2.0, np.float32), 2)
    assert np.allclose(y, 1.0 / (1.0 + math.exp(-2.0)), rtol=1e-15)


# --- whole forward ------------------------------------------------------------


def pin_forward_worked_example(o):
    g = golden("worked_example.json")
    f32 = lambda v: np.array(v, np.float32)
    out, inter = o.forward(f32(g["dense"]), [f32(t) for t in g["tables"]],
                           [np.array(i, np.int64) for i in g["indices"]],
                           [np.array(f, np.int64) for f in g["offsets"]],
                           [f32(w) for w in g["bot_w"]], [f32(b) for b in g["bot_b"]],
                           [f32(w) for w in g["top_w"]], [f32(b) for b in g["top_b"]],
                           ln_bot=g["ln_bot"], ln_top=g["ln_top"], intermediates=True)
    assert np.array_equal(inter["x"], np.array(g["expected_x"], np.float64))
    assert np.array_equal(inter["E"], np.array(g["expected_E"], np.float64))
    assert np.array_equal(inter["R"], np.array(g["expected_R"], np.float64))
    want = np.array([1.0 / (1.0 + math.exp(-a)) for a in g["expected_logits"]])
    np.testing.assert_allclose(out, want, rtol=1e-15, atol=0)


def torch_eager_dlrm_fp64(inp):
    """Independent fp64 PyTorch eager DLRMv1: nn.EmbeddingBag, bmm + tril gather, nn.Linear."""
    w = inp.workload
    with torch.no_grad():
        x = inp.dense.double()
        for W, b in zip(inp.bot_w, inp.bot_b):
            lin = torch.nn.Linear(W.shape[1], W.shape[0]).double()
            lin.weight.copy_(W.double())
            lin.bias.copy_(b.double())
            x = torch.relu(lin(x))
        ly = []
        for tab, idx, off in zip(inp.tables, inp.indices, inp.offsets):
            eb = torch.nn.EmbeddingBag(tab.shape[0], tab.shape[1], mode="sum").double()
            eb.weight.copy_(tab.double())
            ly.append(eb(idx, off))
        S = torch.stack([x] + ly, 1)
        G = torch.bmm(S, S.transpose(1, 2).contiguous())
        li, lj = _tril(w.num_tables + 1)
        R = torch.cat([x, G[:, li, lj]], 1)
        h = R
        n = len(inp.top_w)
        for l, (W, b) in enumerate(zip(inp.top_w, inp.top_b)):
            lin = torch.nn.Linear(W.shape[1], W.shape[0]).double()
            lin.weight.copy_(W.double())
            lin.bias.copy_(b.double())
            h = lin(h)
            h = torch.sigmoid(h) if l == n - 1 else torch.relu(h)
    return h[:, 0].numpy(), R.numpy()


def pin_forward_matches_torch_eager(o):
    import oracle as orc
    cases = [di.make_inputs(di.TINY),
             di.make_inputs(di.custom("pin_small", 24, 5, 5, 40, 8, 3, (5, 16, 8), hidden_top=(16, 8)))]
    # ragged bags, some empty
    w = di.custom("pin_ragged", 17, 3, 3, 30, 4, 1, (3, 4))
    inp = di.make_inputs(w)
    for t in range(w.num_tables):
        off, n = di.ragged_bags(w.batch, 5, 300 + t)
        inp.offsets[t] = off
        inp.indices[t] = torch.randint(0, w.rows, (n,), generator=torch.Generator().manual_seed(400 + t))
    cases.append(inp)
    for inp in cases:
        out, inter = orc.forward_inputs(inp, intermediates=True, oracle=o)
        ref, R = torch_eager_dlrm_fp64(inp)
        np.testing.assert_allclose(inter["R"], R, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def pin_validate_mini_shape(o):
    g = golden("mini_dlrm_shape.json")
    assert o.validate(g["ln_bot"], g["ln_top"], g["n_sparse"], g["m_spa"], g["batch"]) == 0
    assert o.n_pairs(g["n_sparse"] + 1) == g["n_pairs"]
    assert g["ln_top"][0] == g["m_spa"] + g["n_pairs"]
    for name, v in g["invalid_variants"].items():
        assert o.validate(v["ln_bot"], v["ln_top"], g["n_sparse"], g["m_spa"], g["batch"]) != 0, name
    assert o.validate(g["ln_bot"], g["ln_top"], g["n_sparse"], g["m_spa"], 0) != 0


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
