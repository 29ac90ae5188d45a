"""Parity of the HIP path (through the C ABI) with the fp64 oracle on MI355X.

Bars:
* integer / index work bit-exact: the pair-index decoding, bag-size-1 gathers
  (a copy), and bag sums / dots over integer-valued data, whose every partial
  sum is exact in fp32 whatever the order;
* floating point within derived bounds: bag sums within gamma_L * sum|w|,
  dots within gamma_D * sum|u_d v_d|, Linear layers within
  gamma_{K+2} * (|x| |W|^T + |b|) + u |y| (layer-wise: the oracle layer is fed
  the GPU's own fp32 input), with gamma_n = n u / (1 - n u), u = 2^-24;
* the end-to-end sigmoid output within 1e-5 absolute.
Workloads are the seeded synthetic ones of dlrm_inputs at their full sizes,
checked on every output row; for the large ones the oracle reads only the
table rows the batch touches (every output row depends only on its own
sample and the shared weights).
"""
import math

import numpy as np
import pytest
import torch

import dlrm_embedding_interaction_amd as dl
import dlrm_inputs as di
import oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
E2E_TOL = 1e-5


def gamma(n):
    return n * U / (1 - n * U)


def dev():
    return torch.device("cuda", 0)


def log(msg):
    print(msg, flush=True)


def on_gpu(inp):
    return inp.to(dev())


def all_rows(B):
    """Every output row of a batch: the large workloads are checked whole (the
    oracle's samples are independent, so the compact per-sample tables of
    dlrm_inputs.subset keep this affordable), which covers the first and the
    last block of every launch shape, ragged or not."""
    return torch.arange(B)


# --- pair index decoding --------------------------------------------------------


@pytest.mark.parametrize("F", list(range(2, 65)) + [100, 527, 1000, 2049, 4096])
def test_pair_index_map_is_the_nested_loop_order(F):
    i, j = dl.pair_index_map(F)
    ii = i.cpu().numpy()
    jj = j.cpu().numpy()
    want_i = np.repeat(np.arange(F), np.arange(F))
    want_j = np.concatenate([np.arange(r) for r in range(F)])
    assert np.array_equal(ii, want_i) and np.array_equal(jj, want_j)


# --- embedding bags -------------------------------------------------------------


@pytest.mark.parametrize("name", ["tiny", "page4", "manytable"])
def test_embbag_bag1_bitexact(name, orc):
    w = di.get(name)
    log(f"embbag bag1 {name}")
    inp = di.make_inputs(w)
    g = on_gpu(inp)
    E = dl.embbag_sum(g.tables, g.indices, g.offsets)
    torch.cuda.synchronize()
    ref = orc.embbag_sum(inp.tables, inp.indices, inp.offsets)
    assert np.array_equal(E.cpu().double().numpy(), ref)
    # bag size 1 is index_select
    for t in range(w.num_tables):
        assert torch.equal(E[:, t, :], torch.index_select(g.tables[t], 0, g.indices[t]))


@pytest.mark.parametrize("D", [1, 3, 4, 6, 16, 17, 48, 64, 100, 128, 256, 512, 1024])
@pytest.mark.parametrize("L", [1, 20])
def test_embbag_integer_tables_bitexact_all_dims(D, L, orc):
    w = di.custom(f"int_d{D}", 67, 3, 5, 300, D, L, (3, D), cfg_id=11)
    log(f"embbag int D={D} L={L}")
    inp = di.make_inputs(w, int_tables=True)
    g = on_gpu(inp)
    E = dl.embbag_sum(g.tables, g.indices, g.offsets)
    torch.cuda.synchronize()
    assert np.array_equal(E.cpu().double().numpy(), orc.embbag_sum(inp.tables, inp.indices, inp.offsets))


def test_embbag_ragged_and_empty_bags_bitexact(orc):
    T, B, D = 6, 301, 64
    tables, idx, off = [], [], []
    gen = torch.Generator().manual_seed(7)
    for t in range(T):
        o, n = di.ragged_bags(B, 30, 900 + t, empty_frac=0.3)
        tables.append(torch.randint(-8, 9, (97, D), generator=gen).float())
        idx.append(torch.randint(0, 97, (n,), generator=gen))
        off.append(o)
    # a table whose every bag is empty, and one whose bags are all in the last sample
    off[4] = torch.zeros(B, dtype=torch.int64)
    idx[4] = torch.randint(0, 97, (33,), generator=gen)
    off[5] = torch.zeros(B, dtype=torch.int64)
    idx[5] = torch.zeros(0, dtype=torch.int64)
    E = dl.embbag_sum([t.cuda() for t in tables], [i.cuda() for i in idx], [o.cuda() for o in off])
    torch.cuda.synchronize()
    ref = orc.embbag_sum(tables, idx, off)
    assert np.array_equal(E.cpu().double().numpy(), ref)
    ref_t = torch.nn.functional.embedding_bag(idx[0], tables[0], off[0], mode="sum")
    assert torch.equal(E[:, 0].cpu(), ref_t)


def test_embbag_float_multi_hot_within_bound(orc):
    w = di.custom("float_l20", 513, 3, 4, 5000, 128, 20, (3, 128), dist="zipf", cfg_id=12)
    inp = di.make_inputs(w)
    g = on_gpu(inp)
    E = dl.embbag_sum(g.tables, g.indices, g.offsets).cpu().double().numpy()
    ref = orc.embbag_sum(inp.tables, inp.indices, inp.offsets)
    mag = orc.embbag_sum([t.abs() for t in inp.tables], inp.indices, inp.offsets)
    err = np.abs(E - ref)
    assert np.all(err <= gamma(w.bag) * mag + 1e-30), err.max()


def test_embbag_unaligned_tables_take_the_scalar_path(orc):
    gen = torch.Generator().manual_seed(3)
    base = [torch.randint(-8, 9, (200 * 64 + 1,), generator=gen).float() for _ in range(2)]
    tables_cpu = [b[1:].view(200, 64) for b in base]           # 4-byte offset: not 16-byte aligned
    idx = [torch.randint(0, 200, (90,), generator=gen) for _ in range(2)]
    off = [torch.arange(45) * 2 for _ in range(2)]
    tables_gpu = [b.cuda()[1:].view(200, 64) for b in base]
    assert tables_gpu[0].data_ptr() % 16 != 0
    E = dl.embbag_sum(tables_gpu, [i.cuda() for i in idx], [o.cuda() for o in off])
    torch.cuda.synchronize()
    assert np.array_equal(E.cpu().double().numpy(), orc.embbag_sum(tables_cpu, idx, off))


def test_check_indices_counts_bad_data():
    gen = torch.Generator().manual_seed(5)
    idx = [torch.randint(0, 50, (40,), generator=gen).cuda(), torch.randint(0, 60, (40,), generator=gen).cuda()]
    off = [torch.arange(20).cuda() * 2, torch.arange(20).cuda() * 2]
    assert dl.check_indices([50, 60], idx, off) == 0
    idx[0][3] = 50
    idx[1][7] = -2
    off[1][5] = 100          # passes n_indices, and bag 5 > bag 6 start
    assert dl.check_indices([50, 60], idx, off) == 4


# --- interaction ------------------------------------------------------------------


@pytest.mark.parametrize("T,D", [(1, 64), (3, 16), (3, 64), (8, 5), (26, 128), (32, 64), (63, 16), (64, 33)])
@pytest.mark.parametrize("concat", [True, False])
def test_interact_integer_bitexact(T, D, concat, orc):
    B = 129
    gen = torch.Generator().manual_seed(T * 1000 + D)
    x = torch.randint(-16, 17, (B, D), generator=gen).float()
    E = torch.randint(-16, 17, (B, T, D), generator=gen).float()
    out = dl.interact_lower_tri(x.cuda(), E.cuda(), concat_dense=concat)
    torch.cuda.synchronize()
    Z = orc.interact(x.double().numpy(), E.double().numpy())
    want = np.concatenate([x.double().numpy(), Z], 1) if concat else Z
    assert np.array_equal(out.cpu().double().numpy(), want)


@pytest.mark.parametrize("T,D", [(3, 64), (32, 64), (26, 128)])
def test_interact_float_within_bound(T, D, orc):
    B = 1000
    gen = torch.Generator().manual_seed(17)
    x = torch.randn((B, D), generator=gen)
    E = torch.randn((B, T, D), generator=gen)
    out = dl.interact_lower_tri(x.cuda(), E.cuda(), concat_dense=False).cpu().double().numpy()
    Z = orc.interact(x.double().numpy(), E.double().numpy())
    mag = orc.interact(x.abs().double().numpy(), E.abs().double().numpy())
    assert np.all(np.abs(out - Z) <= gamma(D) * mag + 1e-30)


def test_interact_leaves_other_columns_untouched(orc):
    B, T, D = 37, 4, 16
    P = (T + 1) * T // 2
    gen = torch.Generator().manual_seed(9)
    xw = torch.randint(-4, 5, (B, D + 9), generator=gen).float().cuda()
    x = xw[:, 3:3 + D]                              # strided view, ld 25, offset 3
    E = torch.randint(-4, 5, (B, T, D), generator=gen).float().cuda()
    out = torch.full((B, D + P + 7), -777.0, device="cuda")
    dl.interact_lower_tri(x, E, concat_dense=True, out=out)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.all(o[:, D + P:] == -777.0)
    Z = orc.interact(x.cpu().double().numpy(), E.cpu().double().numpy())
    assert np.array_equal(o[:, :D].double().numpy(), x.cpu().double().numpy())
    assert np.array_equal(o[:, D:D + P].double().numpy(), Z)


# --- linear layers --------------------------------------------------------------


def _linear_check(orc, x, W, b, act, y):
    x64 = x.cpu().double().numpy()
    Wc = W.cpu().numpy()
    bc = b.cpu().numpy() if b is not None else None
    ref = orc.linear(x64, Wc, bc, 0)
    mag = np.abs(x64) @ np.abs(Wc.astype(np.float64)).T + (np.abs(bc.astype(np.float64)) if bc is not None else 0)
    K = W.shape[1]
    bound = gamma(K + 2) * mag + U * np.abs(ref) + 1e-30
    got = y.cpu().double().numpy()
    if act == dl.ACT_RELU:
        ref = np.maximum(ref, 0.0)
    if act == dl.ACT_SIGMOID:
        ref = 1.0 / (1.0 + np.exp(-ref))
        bound = 0.25 * bound + 4 * U
    err = np.abs(got - ref)
    assert np.all(err <= bound), (err.max(), (err / bound).max())


SHAPES = [
    (2048, 512, 13), (2048, 256, 512), (2048, 64, 256), (2048, 512, 70), (2048, 512, 592),
    (2048, 1, 256), (8, 32, 4), (8, 16, 32), (8, 32, 22), (8, 1, 32),
    (33, 17, 5), (1, 1, 1), (1, 7, 3), (130, 129, 127), (1000, 300, 200), (4096, 1024, 479), (4096, 128, 256),
    # large-batch tiles: 64x64 of 32x32 blocks for K <= 16, 128x128 otherwise (ragged M, N and K too)
    (16384, 512, 13), (8192, 512, 512), (4100, 1030, 200),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("act", [0, 1, 2])
def test_linear_within_bound(M, N, K, act, orc):
    gen = torch.Generator().manual_seed(M * 7 + N * 13 + K)
    x = torch.randn((M, K), generator=gen)
    W = torch.randn((N, K), generator=gen) * K ** -0.5
    b = torch.randn((N,), generator=gen) * K ** -0.5
    y = dl.linear_bias_act(x.cuda(), W.cuda(), b.cuda(), act)
    torch.cuda.synchronize()
    _linear_check(orc, x, W, b, act, y)


def test_linear_no_bias_and_strided_io(orc):
    gen = torch.Generator().manual_seed(1)
    xw = torch.randn((300, 80), generator=gen).cuda()
    x = xw[:, 5:75]                                  # ld 80, K 70, unaligned start
    W = torch.randn((96, 70), generator=gen).cuda()
    yw = torch.full((300, 100), 5.0, device="cuda")
    y = yw[:, :96]
    dl.linear_bias_act(x, W, None, dl.ACT_NONE, out=y)
    torch.cuda.synchronize()
    assert torch.all(yw[:, 96:] == 5.0)
    _linear_check(orc, x, W, None, 0, y)


def test_linear_strided_unaligned_large_tiles(orc):
    """Row stride 80, a start 5 floats in and K = 70: the scalar-load variants of the 128x128 tiles."""
    gen = torch.Generator().manual_seed(3)
    xw = torch.randn((4200, 80), generator=gen).cuda()
    x = xw[:, 5:75]
    W = (torch.randn((1030, 70), generator=gen) * 70 ** -0.5).cuda()
    b = (torch.randn((1030,), generator=gen) * 70 ** -0.5).cuda()
    yw = torch.full((4200, 1040), 5.0, device="cuda")
    y = yw[:, :1030]
    dl.linear_bias_act(x, W, b, dl.ACT_RELU, out=y)
    torch.cuda.synchronize()
    assert torch.all(yw[:, 1030:] == 5.0)
    _linear_check(orc, x, W, b, dl.ACT_RELU, y)


def test_linear_integer_exact():
    gen = torch.Generator().manual_seed(2)
    x = torch.randint(-3, 4, (257, 70), generator=gen).float()
    W = torch.randint(-3, 4, (130, 70), generator=gen).float()
    b = torch.randint(-3, 4, (130,), generator=gen).float()
    y = dl.linear_bias_act(x.cuda(), W.cuda(), b.cuda(), dl.ACT_RELU).cpu()
    ref = torch.relu(x.double() @ W.double().t() + b.double())
    assert torch.equal(y.double(), ref)


# --- whole forward ------------------------------------------------------------------


def _forward_check(inp_cpu, g, orc, rows=None, tol=E2E_TOL, path="auto"):
    model = dl.Model.from_inputs(g)
    out = model.forward(g.dense, g.indices, g.offsets, path=path)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    if rows is None:
        ref = oracle.forward_inputs(inp_cpu, oracle=orc)
        err = np.abs(got - ref)
    else:
        sub = di.subset(g, rows, compact_tables=True)
        ref = oracle.forward_inputs(sub, oracle=orc)
        err = np.abs(got[rows.numpy()] - ref)
    assert err.max() <= tol, err.max()
    return model, out, err.max()


@pytest.mark.parametrize("path", ["auto", "fused", "layered"])
@pytest.mark.parametrize("name", ["tiny", "page4", "manytable"])
def test_forward_e2e(name, path, orc):
    log(f"forward {name} ({path})")
    inp = di.make_inputs(di.get(name))
    _, _, e = _forward_check(inp, on_gpu(inp), orc, path=path)
    log(f"  max |err| = {e:.3g}")


def test_forward_layerwise_through_standalone_calls(orc):
    """Compose the four calls by hand and check each stage on the GPU's own inputs."""
    inp = di.make_inputs(di.PAGE4)
    g = on_gpu(inp)
    h = g.dense
    for W, b in zip(g.bot_w, g.bot_b):
        y = dl.linear_bias_act(h, W, b, dl.ACT_RELU)
        _linear_check(orc, h, W, b, dl.ACT_RELU, y)
        h = y
    x = h
    E = dl.embbag_sum(g.tables, g.indices, g.offsets)
    assert np.array_equal(E.cpu().double().numpy(), orc.embbag_sum(inp.tables, inp.indices, inp.offsets))
    R = dl.interact_lower_tri(x, E, concat_dense=True)
    Zr = orc.interact(x.cpu().double().numpy(), E.cpu().double().numpy())
    mag = orc.interact(x.abs().cpu().double().numpy(), E.abs().cpu().double().numpy())
    D = x.shape[1]
    assert np.all(np.abs(R[:, D:].cpu().double().numpy() - Zr) <= gamma(D) * mag + 1e-30)
    h = R
    n = len(g.top_w)
    for l, (W, b) in enumerate(zip(g.top_w, g.top_b)):
        act = dl.ACT_SIGMOID if l == n - 1 else dl.ACT_RELU
        y = dl.linear_bias_act(h, W, b, act)
        _linear_check(orc, h, W, b, act, y)
        h = y
    # and the fused forward agrees with the composition
    out = dl.Model.from_inputs(g).forward(g.dense, g.indices, g.offsets)
    assert torch.allclose(out, h[:, 0], atol=1e-6, rtol=0)


@pytest.mark.parametrize("path", ["fused", "layered"])
@pytest.mark.parametrize("B,T", [(16, 1), (16, 32), (64, 8), (256, 4), (2048, 16), (4096, 1), (16384, 8),
                                 (16384, 32),
                                 # the single launch's dots: one MFMA tile per sample from 24 to 32 tables,
                                 # 4x4 register blocks beyond (sweep shapes with other table counts)
                                 (256, 24), (2048, 24), (3000, 32), (64, 40)])
def test_forward_sweep_cells(B, T, path, orc):
    log(f"sweep cell b={B} t={T} ({path})")
    w = di.sweep(B, T)
    g = di.make_inputs(w, device=dev())
    _, _, e = _forward_check(None, g, orc, rows=all_rows(B), path=path)
    log(f"  max |err| over all {B} outputs = {e:.3g}")


def test_forward_stress_full_batch(orc):
    """The 26-table, 1M-row, d=128, bag-20 Zipf workload at full size (13.3 GB of tables),
    every one of its 65536 outputs against the oracle."""
    log("stress: generating 13.3 GB of tables on the GPU")
    g = di.make_inputs(di.STRESS, device=dev())
    rows = all_rows(di.STRESS.batch)
    _, _, e = _forward_check(None, g, orc, rows=rows)
    log(f"  stress max |err| over all {rows.numel()} outputs = {e:.3g}")
    del g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["fused", "layered"])
@pytest.mark.parametrize("B", [1, 2, 3, 5, 17, 100, 2049, 2500])
def test_forward_small_and_ragged_batches(B, path, orc):
    """Batches that leave the last block part-filled; past 2048 the single
    launch holds 16 samples per block."""
    w = di.custom(f"small_b{B}", B, 13, 7, 1000, 64, 1, (13, 64, 64), hidden_top=(64, 32), cfg_id=13)
    inp = di.make_inputs(w)
    _forward_check(inp, on_gpu(inp), orc, path=path)


@pytest.mark.parametrize("path", ["fused", "layered"])
def test_forward_multi_hot_ragged_bags(path, orc):
    w = di.custom("ragged_fwd", 211, 5, 9, 500, 32, 1, (5, 48, 32), hidden_top=(40,), cfg_id=14)
    inp = di.make_inputs(w)
    gen = torch.Generator().manual_seed(21)
    for t in range(w.num_tables):
        off, n = di.ragged_bags(w.batch, 12, 1200 + t, empty_frac=0.25)
        inp.offsets[t] = off
        inp.indices[t] = torch.randint(0, w.rows, (n,), generator=gen)
    _forward_check(inp, on_gpu(inp), orc, path=path)


@pytest.mark.parametrize("path", ["fused", "layered"])
@pytest.mark.parametrize("ln_bot,hidden_top,D", [((13, 37, 16), (), 16), ((3, 300, 100, 48), (129, 17), 48),
                                                 ((70, 1000, 256), (513, 96, 33), 256),
                                                 ((13, 24, 20, 28, 32, 36, 40, 44, 52), (8,) * 7, 52)])
def test_forward_odd_layer_shapes(ln_bot, hidden_top, D, path, orc):
    """Widths that are not multiples of 4 or 16, K tails, a single top layer,
    the widest row of the single-launch path and eight layers per MLP."""
    w = di.custom(f"odd_{len(ln_bot)}_{D}", 77, ln_bot[0], 5, 900, D, 2, ln_bot, hidden_top=hidden_top, cfg_id=22)
    inp = di.make_inputs(w)
    _forward_check(inp, on_gpu(inp), orc, path=path)


@pytest.mark.parametrize("ln_bot,hidden_top,D", [((13, 37, 16), (), 16), ((3, 300, 100, 48), (129, 17), 48),
                                                 ((13, 24, 20, 28, 32, 36, 40, 44, 52), (8,) * 7, 52)])
def test_forward_odd_layer_shapes_sixteen_samples_per_block(ln_bot, hidden_top, D, orc):
    """The same odd widths past batch 2048, where the single launch carries 16
    samples per block (2-step weight rings, partly filled last tiles, waves
    without a tile), and a ragged last block."""
    w = di.custom(f"odd16_{len(ln_bot)}_{D}", 2100, ln_bot[0], 5, 900, D, 2, ln_bot, hidden_top=hidden_top,
                  cfg_id=25)
    inp = di.make_inputs(w)
    _forward_check(inp, on_gpu(inp), orc, path="fused")

@pytest.mark.parametrize("T", [9, 20])
@pytest.mark.parametrize("bag", [1, 2])
@pytest.mark.parametrize("B", [77, 2100])
@pytest.mark.parametrize("ln_bot,hidden_top,D", [((13, 37, 16), (), 16), ((3, 300, 100, 48), (129, 17), 48),
                                                 ((40, 24, 20, 28, 32, 36, 40, 44, 52), (8,) * 7, 52)])
def test_forward_bags_gathered_beside_the_bottom_mlp(ln_bot, hidden_top, D, B, bag, T, orc):
    """From 8 tables the single launch gathers the bags on half its waves while
    the other half runs the bottom MLP: odd widths, a first layer on the vector
    ALUs (13 or 3 inputs) or on the matrix cores (40 inputs), eight bottom
    layers, one- and two-index bags, 8 and 16 samples per block, a ragged last
    block."""
    w = di.custom(f"team_{T}_{len(ln_bot)}_{D}_{bag}", B, ln_bot[0], T, 700, D, bag, ln_bot, hidden_top=hidden_top,
                  cfg_id=28)
    inp = di.make_inputs(w)
    log(f"team T={T} B={B} bag={bag} ln_bot={ln_bot}")
    _forward_check(inp, on_gpu(inp), orc, path="fused")


@pytest.mark.parametrize("T", [3, 9])
@pytest.mark.parametrize("B", [77, 2100])
@pytest.mark.parametrize("n0,n1", [(1, 129), (8, 200), (9, 512), (16, 160), (13, 511)])
def test_forward_first_layer_on_the_matrix_cores(n0, n1, B, T, orc):
    """A first bottom layer of at most 16 inputs and 129-512 outputs runs on the
    matrix cores with its weights requested at kernel start: inputs that fill one
    or two 8-wide chunks, outputs that end inside a 32-wide tile, 8 and 16 samples
    per block (ragged last block), with the bags gathered before it or beside it."""
    w = di.custom(f"first_{n0}_{n1}_{T}", B, n0, T, 700, 32, 1, (n0, n1, 32), hidden_top=(64,), cfg_id=29)
    inp = di.make_inputs(w)
    log(f"first layer {n0}->{n1} T={T} B={B}")
    _forward_check(inp, on_gpu(inp), orc, path="fused")


@pytest.mark.parametrize("T", [3, 5, 7])
@pytest.mark.parametrize("B", [77, 2100])
@pytest.mark.parametrize("bag", ["one", "ragged"])
@pytest.mark.parametrize("ln_bot", [(13, 128, 64), (13, 512, 256, 64), (5, 96, 40, 64)])
def test_forward_bags_gathered_beside_the_last_bottom_layer(ln_bot, bag, B, T, orc):
    """With more bags per block than the gather's lane groups (5-7 tables at 8
    samples per block, 3-7 at 16) and a last bottom layer of at most 64
    outputs, waves 4-7 gather the bags while waves 0-3 run that layer: one-index
    bags and ragged multi-index bags with empty ones, 8 and 16 samples per block
    with a ragged last block; 3 tables at 8 samples per block keep the gather
    before the bottom MLP."""
    w = di.custom(f"late_{T}_{len(ln_bot)}_{bag}", B, ln_bot[0], T, 600, 64, 1, ln_bot, hidden_top=(96,),
                  cfg_id=30)
    inp = di.make_inputs(w)
    if bag == "ragged":
        gen = torch.Generator().manual_seed(31 + T)
        for t in range(T):
            off, n = di.ragged_bags(B, 6, 3100 + 10 * T + t, empty_frac=0.2)
            inp.offsets[t] = off
            inp.indices[t] = torch.randint(0, w.rows, (n,), generator=gen)
    log(f"late gather T={T} B={B} bag={bag} ln_bot={ln_bot}")
    _forward_check(inp, on_gpu(inp), orc, path="fused")


@pytest.mark.parametrize("T", [1, 2, 3])
@pytest.mark.parametrize("B", [77, 2100])
@pytest.mark.parametrize("bag", ["one", "mixed"])
@pytest.mark.parametrize("ln_bot", [(13, 128, 64), (13, 512, 256, 64)])
def test_forward_split_gather(ln_bot, bag, B, T, orc):
    """With one bag slot per lane group, the single launch reads bag bounds and
    indices at kernel start and the rows beside the last bottom layer: bags of
    one index, and (mixed) tables of exactly B indices in empty, one- and
    two-index bags, which the launch cannot tell from one-index bags and which
    take the full gather for their wave; 8 and 16 samples per block, a ragged
    last block."""
    w = di.custom(f"split_{T}_{len(ln_bot)}_{bag}", B, ln_bot[0], T, 500, 64, 1, ln_bot, hidden_top=(80,),
                  cfg_id=31)
    inp = di.make_inputs(w)
    if bag == "mixed":
        gen = torch.Generator().manual_seed(57 + T)
        for t in range(T):
            # lengths 0 / 2 in pairs and 1 elsewhere: B indices in total
            lens = torch.ones(B, dtype=torch.int64)
            pick = torch.randperm(B - 1, generator=gen)[: B // 6]
            lens[pick] = 0
            lens[pick + 1] = lens[pick + 1] + 1
            off = torch.zeros(B, dtype=torch.int64)
            off[1:] = torch.cumsum(lens[:-1], 0)
            inp.offsets[t] = off
            inp.indices[t] = torch.randint(0, w.rows, (int(lens.sum()),), generator=gen)
            assert int(lens.sum()) == B and int(lens.max()) >= 2
    log(f"split gather T={T} B={B} bag={bag} ln_bot={ln_bot}")
    _forward_check(inp, on_gpu(inp), orc, path="fused")



@pytest.mark.parametrize("path", ["fused", "layered"])
def test_forward_zero_last_layer_gives_exactly_half(path):
    inp = di.make_inputs(di.PAGE4)
    inp.top_w[-1].zero_()
    inp.top_b[-1].zero_()
    g = on_gpu(inp)
    out = dl.Model.from_inputs(g).forward(g.dense, g.indices, g.offsets, path=path)
    assert torch.all(out == 0.5)


def test_forward_auto_path_choice():
    """dlrm_forward takes the single launch for the page-4 model, and the layered
    path once the weights no longer fit in L2 (here 4 MB in one top layer), past
    batch 8192, for 32 tables past batch 4096, or without packed weights."""
    g = on_gpu(di.make_inputs(di.PAGE4))
    m = dl.Model.from_inputs(g)
    auto = m.forward(g.dense, g.indices, g.offsets).clone()
    assert torch.equal(auto, m.forward(g.dense, g.indices, g.offsets, path="fused"))
    unpacked = dl.Model.from_inputs(g, pack=False)
    assert torch.equal(unpacked.forward(g.dense, g.indices, g.offsets),
                       m.forward(g.dense, g.indices, g.offsets, path="layered"))
    with pytest.raises(dl.DlrmError) as e:
        unpacked.forward(g.dense, g.indices, g.offsets, path="fused")
    assert e.value.code == dl.DLRM_E_NULL
    cases = [di.custom("big_top", 96, 13, 3, 1000, 64, 1, (13, 64), hidden_top=(1024, 1024), cfg_id=23),
             di.sweep(16384, 1), di.sweep(8192, 32)]
    for w in cases:
        g = on_gpu(di.make_inputs(w))
        m = dl.Model.from_inputs(g)
        auto = m.forward(g.dense, g.indices, g.offsets).clone()
        assert torch.equal(auto, m.forward(g.dense, g.indices, g.offsets, path="layered")), w.name


@pytest.mark.parametrize("T,D", [(64, 64), (2, 1024), (40, 33), (3, 12)])
def test_forward_fused_rejects_what_it_cannot_hold(T, D):
    """Too much LDS (64 tables), rows past 256 or not a multiple of 4, rows under 16."""
    w = di.custom(f"nofuse_{T}_{D}", 16, 5, T, 300, D, 1, (5, 16, D), hidden_top=(32,), cfg_id=24)
    g = on_gpu(di.make_inputs(w))
    with pytest.raises(dl.DlrmError) as e:
        dl.Model.from_inputs(g).forward(g.dense, g.indices, g.offsets, path="fused")
    assert e.value.code == dl.DLRM_E_UNSUPPORTED


def test_forward_rejects_bad_shapes():
    inp = on_gpu(di.make_inputs(di.TINY))
    with pytest.raises(dl.DlrmError) as e:
        dl.Model(inp.tables, inp.bot_w, inp.bot_b, inp.top_w[1:], inp.top_b[1:]).forward(
            inp.dense, inp.indices, inp.offsets)
    assert e.value.code == dl.DLRM_E_SHAPE


@pytest.mark.parametrize("path", ["fused", "layered"])
def test_forward_graph_capture_replays_match_eager(path):
    inp = on_gpu(di.make_inputs(di.PAGE4))
    model = dl.Model.from_inputs(inp)
    B = inp.workload.batch
    out = torch.empty(B, device="cuda")
    ws = model.workspace(B)
    args = model.forward_args(inp.dense, inp.indices, inp.offsets)
    model.forward(inp.dense, inp.indices, inp.offsets, out=out, workspace=ws, args=args, path=path)   # warm up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            model.forward(inp.dense, inp.indices, inp.offsets, out=out, workspace=ws, args=args, path=path)
    torch.cuda.current_stream().wait_stream(s)
    gen = torch.Generator(device="cuda").manual_seed(3)
    for rep in range(4):
        inp.dense.copy_(torch.rand(inp.dense.shape, generator=gen, device="cuda"))
        for t in range(len(inp.indices)):
            inp.indices[t].copy_(torch.randint(0, inp.workload.rows, (B,), generator=gen, device="cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = model.forward(inp.dense, inp.indices, inp.offsets, path=path)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"


# --- fused bag gather + interaction ---------------------------------------------


@pytest.mark.parametrize("T,D,L", [(3, 16, 1), (3, 64, 1), (32, 64, 1), (26, 128, 20), (5, 6, 3), (8, 512, 2),
                                   (28, 48, 1), (24, 80, 3), (33, 64, 1)])
def test_embbag_interact_integer_bitexact(T, D, L, orc):
    w = di.custom(f"fused_{T}_{D}_{L}", 150, 3, T, 400, D, L, (3, D), cfg_id=15)
    inp = di.make_inputs(w, int_tables=True)
    gen = torch.Generator().manual_seed(T + D)
    x = torch.randint(-2, 3, (w.batch, D), generator=gen).float()
    g = on_gpu(inp)
    out = dl.embbag_interact(g.tables, g.indices, g.offsets, x.cuda(), concat_dense=True)
    torch.cuda.synchronize()
    E = orc.embbag_sum(inp.tables, inp.indices, inp.offsets)
    Z = orc.interact(x.double().numpy(), E)
    assert np.array_equal(out.cpu().double().numpy(), np.concatenate([x.double().numpy(), Z], 1))


def test_embbag_interact_in_place_beside_x(orc):
    """x = R[:, :D] and Z written to R[:, D:D+P], the layout the forward uses."""
    inp = di.make_inputs(di.MANYTABLE)
    g = on_gpu(inp)
    B, D, T = 2048, 64, 32
    P = (T + 1) * T // 2
    ld = 596
    gen = torch.Generator().manual_seed(4)
    R = torch.full((B, ld), 123.0, device="cuda")
    x = torch.randn((B, D), generator=gen)
    R[:, :D] = x.cuda()
    dl.embbag_interact(g.tables, g.indices, g.offsets, R, concat_dense=False, out=R[:, D:])
    torch.cuda.synchronize()
    Rc = R.cpu()
    assert torch.equal(Rc[:, :D], x) and torch.all(Rc[:, D + P:] == 123.0)
    E = orc.embbag_sum(inp.tables, inp.indices, inp.offsets)
    Z = orc.interact(x.double().numpy(), E)
    mag = orc.interact(x.abs().double().numpy(), np.abs(E))
    assert np.all(np.abs(Rc[:, D:D + P].double().numpy() - Z) <= gamma(D) * mag + 1e-30)


# --- general bags: mean / max, weights, include_last_offset, padding, int32 ----------


def _general_case(seed, T, B, D, V, max_len, pad_row=3):
    gen = torch.Generator().manual_seed(seed)
    tables, idx, off = [], [], []
    for t in range(T):
        o, n = di.ragged_bags(B, max_len, seed * 10 + t, empty_frac=0.2)
        tables.append(torch.randint(-8, 9, (V, D), generator=gen).float())
        ix = torch.randint(0, V, (n,), generator=gen)
        if n:
            ix[torch.rand(n, generator=gen) < 0.2] = pad_row
        idx.append(ix)
        off.append(o)
    return tables, idx, off


@pytest.mark.parametrize("mode", ["sum", "mean", "max"])
@pytest.mark.parametrize("last", [False, True])
@pytest.mark.parametrize("pad", [None, 3])
@pytest.mark.parametrize("itype", [torch.int64, torch.int32])
@pytest.mark.parametrize("D", [6, 64, 128])
def test_general_bags_integer_tables(mode, last, pad, itype, D, orc):
    """Integer tables: sum and max bit-exact; mean within one fp32 rounding of the exact quotient."""
    T, B = 3, 97
    tables, idx, off = _general_case(31 + D, T, B, D, 50, 24 if D == 128 else 6)
    offs = [torch.cat([o, torch.tensor([i.numel()])]) for o, i in zip(off, idx)] if last else off
    got = dl.embbag([t.cuda() for t in tables], [i.to(itype).cuda() for i in idx], [o.to(itype).cuda() for o in offs],
                    mode=mode, include_last_offset=last, padding_idx=pad)
    torch.cuda.synchronize()
    ref = orc.embbag_ex(tables, idx, offs, mode=mode, include_last_offset=last, padding_idx=pad)
    g = got.cpu().double().numpy()
    if mode == "mean":
        assert np.all(np.abs(g - ref) <= U * np.abs(ref))
    else:
        assert np.array_equal(g, ref)


def test_general_bags_weighted_sum_within_bound(orc):
    T, B, D = 4, 300, 64
    tables, idx, off = _general_case(41, T, B, D, 400, 30)
    gen = torch.Generator().manual_seed(42)
    tables = [torch.randn(t.shape, generator=gen) for t in tables]
    psw = [torch.randn(i.numel(), generator=gen) for i in idx]
    got = dl.embbag([t.cuda() for t in tables], [i.cuda() for i in idx], [o.cuda() for o in off], mode="sum",
                    padding_idx=[3, None, 3, None], per_sample_weights=[w.cuda() for w in psw])
    torch.cuda.synchronize()
    ref = orc.embbag_ex(tables, idx, off, mode="sum", padding_idx=[3, None, 3, None], per_sample_weights=psw)
    mag = orc.embbag_ex([t.abs() for t in tables], idx, off, mode="sum", padding_idx=[3, None, 3, None],
                        per_sample_weights=[w.abs() for w in psw])
    assert np.all(np.abs(got.cpu().double().numpy() - ref) <= gamma(31) * mag + 1e-30)


def test_general_bags_float_mean_and_max_stress_shape(orc):
    """The 26-table, d=128, bag-20 Zipf shape at a reduced batch: max exact, mean within bound."""
    w = di.custom("general_stress", 2048, 13, 26, 100_000, 128, 20, (13, 128), dist="zipf", cfg_id=17)
    inp = di.make_inputs(w)
    g = on_gpu(inp)
    for mode in ("max", "mean"):
        got = dl.embbag(g.tables, g.indices, g.offsets, mode=mode).cpu().double().numpy()
        ref = orc.embbag_ex(inp.tables, inp.indices, inp.offsets, mode=mode)
        if mode == "max":
            assert np.array_equal(got, ref)
        else:
            mag = orc.embbag_ex([t.abs() for t in inp.tables], inp.indices, inp.offsets, mode="mean")
            assert np.all(np.abs(got - ref) <= gamma(21) * mag + 1e-30)


def test_general_sum_equals_plain_bag_sum():
    """With no options the general call is the plain bag sum, bit for bit (int64 and int32 indices)."""
    inp = on_gpu(di.make_inputs(di.custom("gen_plain", 777, 3, 5, 3000, 64, 7, (3, 64), cfg_id=18)))
    plain = dl.embbag_sum(inp.tables, inp.indices, inp.offsets)
    g64 = dl.embbag(inp.tables, inp.indices, inp.offsets)
    g32 = dl.embbag(inp.tables, [i.int() for i in inp.indices], [o.int() for o in inp.offsets])
    assert torch.equal(plain, g64) and torch.equal(plain, g32)


def test_stacked_table_layout_is_bit_identical(orc):
    """One (sum V_t, D) allocation addressed through a base pointer and per-table
    row bases (the stacked layout: dlrm_embbag_sum_stacked, and a model built
    with emb_w NULL) gives the same bags and forward as separate tables, and
    the bags equal the oracle's on integer tables."""
    w = di.custom("stacked", 513, 13, 6, 7000, 64, 2, (13, 64), hidden_top=(64,), cfg_id=19)
    inp = di.make_inputs(w, int_tables=True)
    g = on_gpu(inp)
    stacked = torch.cat(g.tables, 0)
    rows = [w.rows] * w.num_tables
    a = dl.embbag_sum(g.tables, g.indices, g.offsets)
    b = dl.embbag_sum_stacked(stacked, rows, g.indices, g.offsets)
    assert torch.equal(a, b)
    assert np.array_equal(b.cpu().double().numpy(), orc.embbag_sum(inp.tables, inp.indices, inp.offsets))
    # row bases need not be the running sum: the tables in reverse order
    rev = torch.cat(g.tables[::-1], 0)
    base = [(w.num_tables - 1 - t) * w.rows for t in range(w.num_tables)]
    assert torch.equal(a, dl.embbag_sum_stacked(rev, rows, g.indices, g.offsets, row_base=base))
    fl = on_gpu(di.make_inputs(w))
    st = torch.cat(fl.tables, 0)
    for path in ("fused", "layered"):
        fa = dl.Model.from_inputs(fl).forward(fl.dense, fl.indices, fl.offsets, path=path).clone()
        ms = dl.Model(None, fl.bot_w, fl.bot_b, fl.top_w, fl.top_b, n_dense=w.n_dense, stacked=st, rows=rows)
        assert ms._desc.emb_w is None or not bool(ms._desc.emb_w)
        fb = ms.forward(fl.dense, fl.indices, fl.offsets, path=path)
        assert torch.equal(fa, fb)


@pytest.mark.parametrize("name", ["page4", "manytable"])
def test_int32_indices_on_the_hot_path(name, orc):
    """4-byte indices and offsets through dlrm_embbag_sum, dlrm_embbag_interact and
    the forward on both paths: bit for bit the results of 8-byte ones, bags
    bit-exact against the oracle (which widens them exactly), the forward within
    the end-to-end bar."""
    w = di.get(name)
    inp = di.make_inputs(w)
    g = on_gpu(inp)
    i32 = [i.int() for i in g.indices]
    o32 = [o.int() for o in g.offsets]
    E64 = dl.embbag_sum(g.tables, g.indices, g.offsets)
    E32 = dl.embbag_sum(g.tables, i32, o32)
    assert torch.equal(E64, E32)
    assert np.array_equal(E32.cpu().double().numpy(), orc.embbag_sum(inp.tables, inp.indices, inp.offsets))
    x = torch.randn((w.batch, w.dim), generator=torch.Generator().manual_seed(8)).cuda()
    assert torch.equal(dl.embbag_interact(g.tables, g.indices, g.offsets, x),
                       dl.embbag_interact(g.tables, i32, o32, x))
    m = dl.Model.from_inputs(g)
    ref = oracle.forward_inputs(inp, oracle=orc)
    for path in ("auto", "fused", "layered"):
        a = m.forward(g.dense, g.indices, g.offsets, path=path).clone()
        b = m.forward(g.dense, i32, o32, path=path)
        assert torch.equal(a, b), path
        assert np.abs(b.cpu().double().numpy() - ref).max() <= E2E_TOL


def test_int32_ragged_multi_hot_bags_bitexact(orc):
    """Ragged and empty multi-hot bags with 4-byte indices, on integer tables."""
    T, B, D = 5, 301, 128
    tables, idx, off = [], [], []
    gen = torch.Generator().manual_seed(71)
    for t in range(T):
        o, n = di.ragged_bags(B, 30, 700 + t, empty_frac=0.3)
        tables.append(torch.randint(-8, 9, (211, D), generator=gen).float())
        idx.append(torch.randint(0, 211, (n,), generator=gen))
        off.append(o)
    E = dl.embbag_sum([t.cuda() for t in tables], [i.int().cuda() for i in idx], [o.int().cuda() for o in off])
    torch.cuda.synchronize()
    assert np.array_equal(E.cpu().double().numpy(), orc.embbag_sum(tables, idx, off))
    assert dl.check_indices([211] * T, [i.int().cuda() for i in idx], [o.int().cuda() for o in off]) == 0


@pytest.mark.parametrize("T,D,L", [(26, 128, 20), (28, 48, 1), (24, 80, 2), (32, 16, 1), (23, 64, 1)])
def test_forward_fused_gram_dots(T, D, L, orc):
    """Single launch with 24-32 tables: the dots as one 32x32 MFMA tile per sample, over d in
    groups of 64 and a 16-wide tail (D = 48, 80, 16), with multi-hot bags; 23 tables stay on
    the register-block dots."""
    w = di.custom(f"gram_{T}_{D}_{L}", 300, 13, T, 2000, D, L, (13, 64, D), hidden_top=(128,),
                  dist="zipf" if L > 1 else "uniform", cfg_id=25)
    inp = di.make_inputs(w)
    _forward_check(inp, on_gpu(inp), orc, path="fused")


@pytest.mark.parametrize("T,D", [(64, 64), (2, 1024), (40, 33)])
def test_forward_at_the_size_limits(T, D, orc):
    """Most tables (64, so F = 65 and P = 2080), the longest rows (1024) and odd widths."""
    w = di.custom(f"limits_{T}_{D}", 64, 5, T, 300, D, 1, (5, 16, D), hidden_top=(32,), cfg_id=20)
    inp = di.make_inputs(w)
    _forward_check(inp, on_gpu(inp), orc)


# --- bags + interaction as a Gram matrix on the matrix cores (one-index bags) -----


def _int_bags_case(T, D, B, seed, ragged=False, V=300):
    gen = torch.Generator().manual_seed(seed)
    tables, idx, off = [], [], []
    for t in range(T):
        tables.append(torch.randint(-8, 9, (V, D), generator=gen).float())
        if ragged and t % 3 == 1:
            o, n = di.ragged_bags(B, 3, seed * 100 + t, empty_frac=0.3)
        elif ragged and t % 3 == 2:
            # one index per bag except a few empty bags
            lens = torch.ones(B, dtype=torch.int64)
            lens[torch.rand(B, generator=gen) < 0.1] = 0
            o = torch.zeros(B, dtype=torch.int64)
            o[1:] = torch.cumsum(lens[:-1], 0)
            n = int(lens.sum())
        else:
            o, n = torch.arange(B, dtype=torch.int64), B
        idx.append(torch.randint(0, V, (n,), generator=gen))
        off.append(o)
    x = torch.randint(-8, 9, (B, D), generator=gen).float()
    return tables, idx, off, x


@pytest.mark.parametrize("T,D,B", [
    # one 16x16 tile (F <= 16), then one tile plus the 17th feature, three tiles, three plus the 33rd
    (1, 64, 4100), (4, 64, 4100), (8, 64, 4100), (15, 64, 4100), (16, 64, 4100), (17, 64, 4100),
    (24, 64, 4100), (31, 64, 4100), (32, 64, 4100),
    # rows of 32 and 128 floats
    (8, 32, 3000), (16, 32, 3000), (32, 32, 3000), (8, 128, 3000), (16, 128, 3000), (20, 128, 3000),
    (32, 128, 3000),
    # samples per wave 1, 4 and 8, each with a partly filled last wave
    (32, 64, 37), (32, 64, 9001), (32, 64, 16500), (8, 64, 20003),
])
@pytest.mark.parametrize("itype", [torch.int64, torch.int32])
def test_gram_interaction_integer_bitexact(T, D, B, itype, orc):
    """Integer tables and x: every bag sum and dot is exact in fp32, so the Gram
    kernel must equal the oracle bit for bit, x columns included."""
    tables, idx, off, x = _int_bags_case(T, D, B, seed=T * 131 + D + B)
    log(f"gram T={T} D={D} B={B} {itype}")
    out = dl.embbag_interact([t.cuda() for t in tables], [i.to(itype).cuda() for i in idx],
                             [o.to(itype).cuda() for o in off], x.cuda(), concat_dense=True)
    torch.cuda.synchronize()
    E = orc.embbag_sum(tables, idx, off)
    Z = orc.interact(x.double().numpy(), E)
    assert np.array_equal(out.cpu().double().numpy(), np.concatenate([x.double().numpy(), Z], 1))


@pytest.mark.parametrize("T,D,B", [(8, 64, 3001), (16, 64, 700), (32, 64, 5000), (32, 128, 1100)])
def test_gram_interaction_ragged_bags_bitexact(T, D, B, orc):
    """Empty bags on the fast path, and bags of 2-3 indices that send their waves
    down the general path; Z written beside x in one buffer, as the forward does."""
    tables, idx, off, x = _int_bags_case(T, D, B, seed=7 * T + D, ragged=True)
    P = (T + 1) * T // 2
    ld = (D + P + 3) // 4 * 4 + 4
    R = torch.full((B, ld), 99.0)
    R[:, :D] = x
    Rg = R.cuda()
    dl.embbag_interact([t.cuda() for t in tables], [i.cuda() for i in idx], [o.cuda() for o in off], Rg,
                       concat_dense=False, out=Rg[:, D:])
    torch.cuda.synchronize()
    Rc = Rg.cpu()
    E = orc.embbag_sum(tables, idx, off)
    Z = orc.interact(x.double().numpy(), E)
    assert torch.equal(Rc[:, :D], x) and torch.all(Rc[:, D + P:] == 99.0)
    assert np.array_equal(Rc[:, D:D + P].double().numpy(), Z)


@pytest.mark.parametrize("T,D", [(8, 64), (16, 64), (32, 64), (26, 128)])
def test_gram_interaction_float_within_bound(T, D, orc):
    """Random fp32 tables and x at batch 8192: every dot within gamma_D sum |u_d v_d|."""
    B = 8192
    w = di.custom(f"gramf_{T}_{D}", B, 3, T, 5000, D, 1, (3, D), cfg_id=27)
    inp = di.make_inputs(w)
    g = on_gpu(inp)
    x = torch.randn((B, D), generator=torch.Generator().manual_seed(T))
    out = dl.embbag_interact(g.tables, g.indices, g.offsets, x.cuda(), concat_dense=False).cpu().double().numpy()
    E = orc.embbag_sum(inp.tables, inp.indices, inp.offsets)
    Z = orc.interact(x.double().numpy(), E)
    mag = orc.interact(x.abs().double().numpy(), np.abs(E))
    assert np.all(np.abs(out - Z) <= gamma(D) * mag + 1e-30)
