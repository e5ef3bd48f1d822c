"""GPU parity at the full workload sizes, for the three weight forms.

decode T=128 and T=256, prefill T=8192, skewed prefill T=16384 and skewed
decode T=256 (H=6144, I=2048, E=256, top-8; the skewed routings Zipf(1.1),
where the hottest expert gets most of the tokens), each with the group-128 INT4 x FP8 experts, the
per-channel INT4 x INT8 ones and the MXFP4 ones.  The layer runs on the GPU
as the benchmark runs it (prepacked experts, automatic kernel choice, fused
SwiGLU, the one-launch front at decode), once per workload and form, and
every buffer it wrote is compared:
  * routing, permutation and the quantized activations: every token,
    bit-exact;
  * the gate/up GEMM, launched unfused at full size on the layer's own
    inputs (h), and the layer's down GEMM (o): every routed row at decode;
    at prefill every row of six whole experts (the first and last with rows,
    the hottest, the smallest, one cut into two or three equal-height tiles,
    and a seeded random one), against the oracle fed the same inputs, to
    the GEMM bar;
  * the layer's fused gate/up launch (act): SwiGLU of the GPU's own gate/up
    values to a few fp32 ulp per element, and the oracle's act to the tight
    Frobenius bar.  (SwiGLU can amplify a gate value's relative error many
    times where its 6144-term sum nearly cancels, so the per-element bar is
    held by the GEMM output h and the epilogue is checked on its own);
  * the re-quantized activations: the GPU's codes and scales are exactly the
    quantization of its own act; the codes that differ from an independent
    oracle run (the two sides' act differ by GEMM rounding) are counted;
  * the down GEMM against that independent run, per element on the rows
    with no differing code;
  * the layer output against an independent oracle run: every token at
    decode, a seeded sample of tokens at prefill (the layer is token-local),
    with the bars of check_layer_output.
The unfused GEMM calls of both kernels are also run on sampled rows at the
full K.  The oracle's GEMMs run on threads, one expert at a time
(oracle_par); the numbers of differing codes are printed per workload.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle_par
from gpu_util import (GEMM_FRO_TIGHT, assert_float_parity, bf16_to_dev, check_layer_output, check_requant,
                      check_swiglu_epilogue, host, near_midpoint, say, to_dev)
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE, W4A8MoEChannel, W4A8MoEMxfp4

pytestmark = pytest.mark.gpu

CONFIGS = [1, 2, 3, 4, "skewed-decode"]
FORMS = ["g128", "channel", "mxfp4"]
LAYERS = {"g128": W4A8MoE, "channel": W4A8MoEChannel, "mxfp4": W4A8MoEMxfp4}


_workload = {}


def _workload_of(index):
    """The seeded workload of a config, kept while its forms run (one config held at a time)."""
    if index not in _workload:
        _workload.clear()
        say(f"generate config {index}")
        _workload[index] = workloads.make_skewed_decode() if index == "skewed-decode" else workloads.make_config(index)
    return _workload[index]


# workload-major order: each workload's 5 GB of experts is drawn once for its three forms
@pytest.fixture(scope="module", params=[(c, f) for c in CONFIGS for f in FORMS], ids=lambda p: f"{p[0] if isinstance(p[0], str) else f'config{p[0]}'}-{p[1]}")
def run(request):
    index, form = request.param
    wl = _workload_of(index)
    if form == "g128":
        weights = (wl.w13, wl.s13, wl.w2, wl.s2)
    elif form == "channel":
        cs13, cs2 = workloads.channel_scales(wl)
        weights = (wl.w13, cs13, wl.w2, cs2)
    else:
        weights = workloads.mxfp4_weights(wl)
    torch.cuda.empty_cache()
    moe = LAYERS[form](*(to_dev(t) for t in weights), k=wl.shape.k)
    say(f"forward {wl.shape.name} ({form})")
    y = moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits))
    b = moe.buffers(wl.shape.T)
    # the unfused gate/up GEMM, launched at full size on the layer's own inputs (automatic kernel choice)
    R = wl.shape.T * wl.shape.k
    say(f"unfused gate/up GEMM {wl.shape.name} ({form})")
    if form == "g128":
        h = ops.w4a8_moe_grouped_gemm_prepacked(b["qx"], b["sx"], b["row_token"], b["offsets"], moe.w13, moe.s13, R)
    elif form == "channel":
        h = ops.w4a8_moe_grouped_gemm_i8_prepacked(b["qx"], b["sx"], b["rx"], b["row_token"], b["offsets"], moe.w13,
                                                   moe.s13, M_total=R)
    else:
        h = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(b["qx"], b["sx"], b["row_token"], b["offsets"], moe.w13,
                                                      moe.s13, R)
    got = {k: host(v) for k, v in b.items() if k not in ("workspace", "counter")}
    got["y"] = host(y)
    got["h"] = host(h)
    del h
    r = dict(form=form, wl=wl, weights=weights, moe=moe, got=got, cache={})
    yield r
    r.clear()
    del moe, y
    torch.cuda.empty_cache()
    if index == CONFIGS[-1] and form == FORMS[-1]:
        _workload.clear()


def _decode(wl):
    return wl.shape.T <= 256


def _experts_to_check(wl, offsets):
    """All experts at decode; six whole experts at prefill."""
    counts = np.diff(offsets)
    nonempty = np.nonzero(counts)[0]
    if _decode(wl):
        return nonempty
    pick = {int(nonempty[0]), int(nonempty[-1]), int(np.argmax(counts)),
            int(nonempty[np.argmin(counts[nonempty])])}
    multi = [int(e) for e in nonempty if 256 < counts[e] <= 768 and int(e) not in pick]
    if multi:
        pick.add(multi[len(multi) // 2])          # two or three square tiles of equal height
    rng = np.random.Generator(np.random.PCG64(500 + wl.shape.T))
    rest = [int(e) for e in nonempty if int(e) not in pick]
    pick.add(int(rng.choice(rest)))
    return np.array(sorted(pick))


def _oracle_front(r):
    """The oracle's steps 1-3 on every token (computed once per workload and form)."""
    if "front" not in r["cache"]:
        wl, form = r["wl"], r["form"]
        qx, sx = oracle_par.FORMS[form][0](wl.x_bf16)
        ids, w = oracle.route(wl.logits, wl.shape.k)
        offsets, row_token, inv_pos = oracle.permute(ids, wl.shape.E)
        r["cache"]["front"] = dict(qx=qx, sx=sx, ids=ids, w=w, offsets=offsets, row_token=row_token, inv_pos=inv_pos)
    return r["cache"]["front"]


def _oracle_rows(r):
    """An independent oracle run on the checked experts' rows (from the oracle's own steps 1-3), plus the
    oracle's down GEMM on the GPU's re-quantized activations of those rows."""
    if "rows" in r["cache"]:
        return r["cache"]["rows"]
    form, wl, got = r["form"], r["wl"], r["got"]
    w13, s13, w2, s2 = r["weights"]
    requant = oracle_par.FORMS[form][1]
    f = _oracle_front(r)
    offsets = f["offsets"]
    experts = _experts_to_check(wl, offsets)
    say(f"{wl.shape.name} ({form}): oracle gate/up GEMM on {len(experts)} experts")
    h = oracle_par.gemm_experts(form, f["qx"], f["sx"], f["row_token"], offsets, w13, s13, experts)
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in experts])
    a32 = np.zeros_like(h[:, : h.shape[1] // 2])
    a32[rows] = oracle.swiglu_f32(h[rows])
    qa = np.zeros(a32.shape, got["qa"].dtype)
    sa = np.ones(a32.shape[0], np.float32)
    qa[rows], sa[rows] = requant(a32[rows])
    say(f"{wl.shape.name} ({form}): oracle down GEMM on the GPU's and on the oracle's codes")
    o_same = oracle_par.gemm_experts(form, got["qa"], got["sa"], None, offsets, w2, s2, experts)
    o_indep = oracle_par.gemm_experts(form, qa, sa, None, offsets, w2, s2, experts)
    res = dict(experts=experts, rows=rows, h=h, a32=a32, qa=qa, sa=sa, o_same=o_same, o_indep=o_indep)
    r["cache"]["rows"] = res
    return res


def test_front(run):
    """Routing, permutation and quantized activations of every token: bit-exact."""
    wl, got, form = run["wl"], run["got"], run["form"]
    sh = wl.shape
    f = _oracle_front(run)
    assert np.array_equal(got["ids"], f["ids"])
    assert np.all(np.abs(got["w"].astype(np.float64) - f["w"]) <= 1e-6 * np.abs(f["w"]))
    for name in ("offsets", "row_token", "inv_pos", "qx"):
        assert np.array_equal(got[name], f[name]), name
    assert np.array_equal(got["sx"].view(np.uint32), f["sx"].view(np.uint32))
    if form == "channel":
        assert np.array_equal(got["rx"], oracle.code_row_sums(f["qx"]))
    counts = np.diff(f["offsets"])
    say(f"{sh.name} ({form}): touched {int((counts > 0).sum())} experts, rows per expert "
        f"{int(counts[counts > 0].min())}..{int(counts.max())}, empty {int((counts == 0).sum())}")
    if sh.zipf_s is not None:
        assert (counts == 0).sum() >= 1                # the skew leaves some experts empty


def test_gemm_rows(run):
    """h, act and o of full-size launches on every checked row, and the re-quantized codes."""
    wl, got, form = run["wl"], run["got"], run["form"]
    res = _oracle_rows(run)
    rows = res["rows"]
    name = f"{wl.shape.name} ({form})"
    fro = 1e-5 if form == "channel" else GEMM_FRO_TIGHT
    # the gate/up GEMM (unfused launch) on the same inputs: the GEMM bar on every element
    r_h = assert_float_parity(got["h"][rows], res["h"][rows], f"{name} h", fro_tight=fro)
    # the layer's fused launch: SwiGLU of those gate/up values, to a few ulp; and against the oracle
    ulps = check_swiglu_epilogue(got["act"][rows], got["h"][rows], f"{name} act")
    fro_act = np.linalg.norm(got["act"][rows] - res["a32"][rows]) / np.linalg.norm(res["a32"][rows])
    assert fro_act <= fro, fro_act
    assert np.array_equal(got["pmax"][rows].max(axis=1), np.abs(got["act"][rows]).max(axis=1))
    # re-quantization: exact on the GPU's own act; the codes that differ from the independent run
    flipped = check_requant(got["act"][rows], got["qa"][rows], got["sa"][rows], res["qa"][rows],
                            int8=form == "channel")
    if form == "channel":
        assert np.array_equal(got["ra"][rows], oracle.code_row_sums(got["qa"][rows]))
    n_flip = int(flipped.sum())
    assert n_flip <= 1e-2 * flipped.size, n_flip
    # the layer's down GEMM on the same inputs
    r_o = assert_float_parity(got["o"][rows], res["o_same"][rows], f"{name} o", fro_tight=fro)
    # and against the independent run: per element on the rows with no differing code
    clean = ~flipped.any(axis=1)
    r_ind = assert_float_parity(got["o"][rows][clean], res["o_indep"][rows][clean], f"{name} o vs independent oracle")
    # (over all rows, flips included, this is reported only: o is an intermediate, and the 2e-3
    # bar of the layer applies to its output, test_end_to_end)
    fro_all = np.linalg.norm(got["o"][rows] - res["o_indep"][rows]) / np.linalg.norm(res["o_indep"][rows])
    counts = np.diff(got["offsets"])
    say(f"{name}: {rows.size} rows of {len(res['experts'])} experts "
        f"(rows per expert {sorted(int(counts[e]) for e in res['experts'])}); "
        f"h {r_h}; act within {ulps:.1f} ulp of SwiGLU(h), fro vs oracle {fro_act:.2e}; o {r_o}; "
        f"codes differing from the independent run {n_flip} of {flipped.size} in {int((~clean).sum())} rows; "
        f"o vs independent on the other rows {r_ind}, all rows fro {fro_all:.2e}")


def test_end_to_end(run):
    """The layer output against an independent oracle run."""
    wl, got, form = run["wl"], run["got"], run["form"]
    sh = wl.shape
    w13, s13, w2, s2 = run["weights"]
    k = sh.k
    if _decode(wl):
        # every token: the independent run of the row test covers every routed row
        f, res = _oracle_front(run), _oracle_rows(run)
        assert res["rows"].size == sh.T * k
        flipped = check_requant(got["act"], got["qa"], got["sa"], res["qa"], int8=form == "channel")
        row_flip = flipped.any(axis=1)
        token_flipped = row_flip[f["inv_pos"]].reshape(sh.T, k).any(axis=1)
        y_indep = oracle.unpermute(res["o_indep"], f["inv_pos"], f["w"])
        y_same = oracle.unpermute(res["o_same"], f["inv_pos"], f["w"])
        r = check_layer_output(got["y"], y_indep, y_same, token_flipped, f"{sh.name} ({form}) output")
        say(f"{sh.name} ({form}) output, every token: {r}; {int(flipped.sum())} differing codes in "
            f"{int(row_flip.sum())} of {row_flip.size} routed rows")
        return
    rng = np.random.Generator(np.random.PCG64(600 + sh.T))
    hot = int(np.argmax(np.diff(got["offsets"])))
    hot_token = int(got["row_token"][got["offsets"][hot]])
    sel = np.unique(np.concatenate([[0, sh.T - 1, hot_token], rng.integers(0, sh.T, size=5)]))
    say(f"{sh.name} ({form}): independent oracle layer on {sel.size} tokens")
    res = oracle_par.layer(form, wl.x_bf16[sel], wl.logits[sel], w13, s13, w2, s2, k=sh.k)
    # the GPU's routed rows of these tokens, in the oracle run's row order
    gpu_rows = np.empty(sel.size * k, np.int64)
    for i, t in enumerate(sel):
        gpu_rows[res["inv_pos"][i * k:(i + 1) * k]] = got["inv_pos"][t * k:(t + 1) * k]
    flipped = check_requant(got["act"][gpu_rows], got["qa"][gpu_rows], got["sa"][gpu_rows], res["qa"],
                            int8=form == "channel")
    row_flip = flipped.any(axis=1)
    token_flipped = row_flip[res["inv_pos"]].reshape(sel.size, k).any(axis=1)
    # the oracle's down GEMM and combine on the GPU's (checked) codes
    o_same = oracle_par.gemm_experts(form, got["qa"][gpu_rows], got["sa"][gpu_rows], None, res["offsets"], w2, s2)
    y_same = oracle.unpermute(o_same, res["inv_pos"], res["w"])
    r = check_layer_output(got["y"][sel], res["y"], y_same, token_flipped, f"{sh.name} ({form}) output")
    say(f"{sh.name} ({form}) output: {r}; {int(flipped.sum())} differing codes in {int(row_flip.sum())} of "
        f"{row_flip.size} routed rows")


def test_unfused_calls_sampled_rows(run):
    """The unfused gate/up GEMM (both kernels), SwiGLU and down GEMM at the full K on sampled rows."""
    wl, got, form, moe = run["wl"], run["got"], run["form"], run["moe"]
    sh = wl.shape
    w13, s13, w2, s2 = run["weights"]
    offsets = got["offsets"]
    rng = np.random.Generator(np.random.PCG64(100 + sh.T))
    counts = np.diff(offsets)
    nonempty = np.nonzero(counts)[0]
    experts = sorted({int(nonempty[0]), int(nonempty[-1]), int(np.argmax(counts))}
                     | {int(e) for e in rng.choice(nonempty, size=3, replace=False)})
    P = np.array(sorted({int(p) for e in experts for p in (offsets[e], offsets[e + 1] - 1,
                                                           (offsets[e] + offsets[e + 1]) // 2)}))
    ex_of = np.searchsorted(offsets, P, side="right") - 1
    sub = np.zeros(sh.E + 1, np.int32)
    np.add.at(sub, ex_of + 1, 1)
    sub = np.cumsum(sub).astype(np.int32)
    quant, requant, _ = oracle_par.FORMS[form]
    qx, sx = quant(wl.x_bf16[got["row_token"][P]])
    h = oracle_par.gemm_experts(form, qx, sx, None, sub, w13, s13)
    fro = 1e-5 if form == "channel" else GEMM_FRO_TIGHT
    rsum = oracle.code_row_sums(qx) if form == "channel" else None
    for algo in (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED):
        say(f"{sh.name} ({form}): unfused gate/up GEMM on {P.size} rows algo={algo}")
        if form == "g128":
            gh = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(qx), to_dev(sx), None, to_dev(sub), moe.w13, moe.s13,
                                                     P.size, algo=algo)
        elif form == "channel":
            gh = ops.w4a8_moe_grouped_gemm_i8_prepacked(to_dev(qx), to_dev(sx), to_dev(rsum), None, to_dev(sub),
                                                        moe.w13, moe.s13, M_total=P.size, algo=algo)
        else:
            gh = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(qx), to_dev(sx), None, to_dev(sub), moe.w13,
                                                           moe.s13, P.size, algo=algo)
        assert_float_parity(host(gh), h, f"{sh.name} ({form}) gate/up algo={algo}", fro_tight=fro)
    a32 = oracle.swiglu_f32(h)
    qa, sa = requant(a32)
    # the unfused SwiGLU on the oracle's h: scales within 1e-6, codes equal except where the
    # oracle's quotient lies at a rounding midpoint (within 1e-5 relative)
    say(f"{sh.name} ({form}): swiglu on {P.size} oracle rows")
    if form == "channel":
        gq, gs, gr = (host(t) for t in ops.w4a8_moe_swiglu_i8(to_dev(h)))
        assert np.array_equal(gr, oracle.code_row_sums(gq))
        q = a32.astype(np.float64) / sa.astype(np.float64)[:, None]
        near = np.abs(np.abs(q - np.floor(q)) - 0.5) < 1e-5 * np.maximum(np.abs(q), 1.0)
    else:
        gq, gs = (host(t) for t in ops.w4a8_moe_swiglu(to_dev(h)))
        near = near_midpoint(a32, sa)
    assert np.all(np.abs(gs.astype(np.float64) - sa) <= 1e-6 * sa)
    diff = gq != qa
    assert np.all(near[diff]), f"{int((diff & ~near).sum())} codes differ away from a rounding midpoint"
    o = oracle_par.gemm_experts(form, qa, sa, None, sub, w2, s2)
    for algo in (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED):
        say(f"{sh.name} ({form}): down GEMM on {P.size} oracle rows algo={algo}")
        if form == "g128":
            go = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(qa), to_dev(sa), None, to_dev(sub), moe.w2, moe.s2,
                                                     P.size, algo=algo)
        elif form == "channel":
            go = ops.w4a8_moe_grouped_gemm_i8_prepacked(to_dev(qa), to_dev(sa), to_dev(oracle.code_row_sums(qa)),
                                                        None, to_dev(sub), moe.w2, moe.s2, M_total=P.size,
                                                        algo=algo)
        else:
            go = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(qa), to_dev(sa), None, to_dev(sub), moe.w2,
                                                           moe.s2, P.size, algo=algo)
        assert_float_parity(host(go), o, f"{sh.name} ({form}) down algo={algo}", fro_tight=fro)


def test_scatter_chain(run):
    """Step 7 as a scatter from the down GEMM, at full size on the layer's own buffers: the row sources
    invert the permutation exactly, the scatter GEMM's rows are bit for bit the plain GEMM's (same codes,
    same scales row_scale = sa w, the same automatic kernel choice), and the contiguous combine gives the
    layer's gather output (checked against the oracle above) up to one more fp32 rounding per term."""
    wl, got, form, moe = run["wl"], run["got"], run["form"], run["moe"]
    sh = wl.shape
    b = moe.buffers(sh.T)
    R = sh.T * sh.k
    say(f"{sh.name} ({form}): scatter chain")
    row_src, row_scale = ops.w4a8_moe_row_sources(b["inv_pos"], b["w"], b["sa"], R)
    inv = got["inv_pos"]
    want_src = np.empty(R, np.int32)
    want_src[inv] = np.arange(R, dtype=np.int32)
    assert np.array_equal(host(row_src), want_src)
    o_tok = torch.empty((R, sh.H), dtype=torch.float32, device="cuda:0")
    if form == "channel":
        plain = ops.w4a8_moe_grouped_gemm_i8_prepacked(b["qa"], row_scale, b["ra"], None, b["offsets"], moe.w2,
                                                       moe.s2, M_total=R)
        ops.w4a8_moe_grouped_gemm_scatter_i8_prepacked(b["qa"], row_scale, b["ra"], None, b["offsets"], moe.w2,
                                                       moe.s2, R, row_src, o_tok)
    else:
        plain = moe.GEMM(b["qa"], row_scale, None, b["offsets"], moe.w2, moe.s2, R)
        moe.GEMM_SCATTER(b["qa"], row_scale, None, b["offsets"], moe.w2, moe.s2, R, row_src, o_tok)
    # every row of the scatter output against the plain GEMM's row, compared on the device
    same = torch.equal(o_tok.index_select(0, row_src.long()).view(torch.int32), plain.view(torch.int32))
    del plain
    assert same, "scatter rows differ from the plain GEMM's"
    y = host(ops.w4a8_moe_combine(o_tok, b["inv_pos"], sh.T, sh.k))
    del o_tok
    r = assert_float_parity(y, got["y"], f"{sh.name} ({form}) scatter vs gather output", fro_tight=1e-6)
    say(f"{sh.name} ({form}) scatter chain output vs the gather output: {r}")
