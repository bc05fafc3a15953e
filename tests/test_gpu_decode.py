"""GPU decode-side reductions (dllm_decode_commit, dllm_decode_verify and their
pieces) against the oracle (oracle/decode.py).

Bars:
  * token: bit-exact (the maximum of bf16 or fp32 inputs involves no rounding;
    ties go to the lowest id on both sides);
  * confidence: relative 1e-4 against the fp64 oracle.  The kernel sums up to
    a few hundred exp terms per lane in fp32 and merges lanes and splits in a
    fixed tree; with the hardware exp2 (about 1 ulp) the worst-case relative
    error at 128 Ki tokens is a few 1e-5;
  * decisions (commit / accept flags and counts): bit-exact against the
    oracle's rule applied to the kernel's own fp32 confidences and the fp32
    threshold, so both sides decide in the same precision.

Inputs: seeded synthetic logits, N(0,1) background with one planted peak per
row whose height spreads the confidence over about 0.1 .. 0.99 (some rows
carry a twin peak of equal height to exercise the tie rule), at the assumed
LM-head width of 128 Ki tokens and at small, ragged widths.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

EPS, GAMMA = 0.9, 0.8
F32_EPS, F32_GAMMA = float(np.float32(EPS)), float(np.float32(GAMMA))

CASES = [
    # (sequence lengths, vocab, dtype, row stride (None: dense), twin fraction)
    ([32], W.VOCAB, "bf16", None, 0.1),              # one sequence's masked window, split rows
    ([5, 0, 17, 1], 1000, "bf16", None, 0.3),        # vector loads, ragged tail of 0 (1000 % 8 == 0)
    ([3, 9], 4099, "bf16", 4104, 0.3),               # ragged width, aligned stride: vectors + tail
    ([4, 2], 4099, "bf16", None, 0.3),               # unaligned rows: scalar loads
    ([2, 7], 50001, "f32", None, 0.2),               # fp32, scalar loads
    ([6], 65539, "f32", 65540, 0.2),                 # fp32 vectors + tail, split rows
    ([1, 1], 1, "bf16", None, 0.0),                  # one-token vocabulary: confidence 1
    ([40, 3], 262147, "bf16", 262152, 0.5),          # wide rows, many splits, tie-heavy
]


def _dev(a, gpu):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu)


def _logits(case, seed, gpu):
    import torch
    lens, V, dt, stride, twin = case
    rows = W.decode_rows(seed, lens, V, twin_frac=twin)
    host = W.decode_logits_host(seed, rows, V, dt)
    R = host.shape[0]
    S = stride or V
    if dt == "bf16":
        ref = W.bf16_bits_to_f64(host)
        buf = torch.zeros((R, S), dtype=torch.int16)
        buf[:, :V] = torch.from_numpy(host.view(np.int16))
        dev = buf.view(torch.bfloat16).to(gpu)
    else:
        ref = host.astype(np.float64)
        buf = torch.zeros((R, S), dtype=torch.float32)
        buf[:, :V] = torch.from_numpy(host)
        dev = buf.to(gpu)
    return rows, ref, dev


def _alloc(R, n_seq, V, gpu):
    import torch
    from io_aware_kv_amd import dllm
    ws_bytes = dllm.confidence_workspace(R, V)
    return dict(
        token=torch.full((R,), -7, dtype=torch.int32, device=gpu),
        conf=torch.full((R,), -1.0, dtype=torch.float32, device=gpu),
        flag=torch.full((R,), 7, dtype=torch.uint8, device=gpu),
        count=torch.full((n_seq,), -7, dtype=torch.int32, device=gpu),
        ws=torch.empty(max(ws_bytes, 16) // 4 + 4, dtype=torch.float32, device=gpu),
    )


def _check_rows(tok, conf, ref):
    o_tok, o_conf = O.confidence_argmax(ref)
    assert np.array_equal(tok, o_tok), np.flatnonzero(tok != o_tok)[:10]
    np.testing.assert_allclose(conf, o_conf, rtol=1e-4, atol=0)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[2]}-V{c[1]}-{len(c[0])}seq" for c in CASES])
def test_decode_commit_matches_oracle(case, gpu):
    import torch
    from io_aware_kv_amd import dllm
    lens, V, dt, stride, twin = case
    print(f"[gpu] decode_commit lens={lens} V={V} {dt} stride={stride}", flush=True)
    rows, ref, dev = _logits(case, 3, gpu)
    R = ref.shape[0]
    cu = _dev(rows.cu, gpu)
    b = _alloc(R, len(lens), V, gpu)
    dllm.decode_commit(dev, cu, EPS, b["token"], b["conf"], b["flag"], b["count"], b["ws"], vocab=V)
    torch.cuda.synchronize()
    tok, conf = b["token"].cpu().numpy(), b["conf"].cpu().numpy()
    _check_rows(tok, conf, ref)
    commit, n = O.confidence_commit(conf.astype(np.float64), rows.cu, F32_EPS)
    assert np.array_equal(b["flag"].cpu().numpy().astype(bool), commit)
    assert np.array_equal(b["count"].cpu().numpy(), n)
    # the standalone pieces give the same results
    t2, c2 = torch.empty_like(b["token"]), torch.empty_like(b["conf"])
    dllm.confidence_argmax(dev, t2, c2, b["ws"], vocab=V)
    f2, n2 = torch.full_like(b["flag"], 7), torch.full_like(b["count"], -7)
    dllm.confidence_commit(cu, c2, EPS, f2, n2)
    torch.cuda.synchronize()
    assert torch.equal(t2, b["token"]) and torch.equal(c2, b["conf"])
    assert torch.equal(f2, b["flag"]) and torch.equal(n2, b["count"])


@pytest.mark.parametrize("case", CASES[:6], ids=[f"{c[2]}-V{c[1]}-{len(c[0])}seq" for c in CASES[:6]])
def test_decode_verify_matches_oracle(case, gpu):
    import torch
    from io_aware_kv_amd import dllm
    lens, V, dt, stride, twin = case
    print(f"[gpu] decode_verify lens={lens} V={V} {dt} stride={stride}", flush=True)
    rows, ref, dev = _logits(case, 4, gpu)
    R = ref.shape[0]
    cu = _dev(rows.cu, gpu)
    draft = _dev(rows.draft, gpu)
    b = _alloc(R, len(lens), V, gpu)
    dllm.decode_verify(dev, cu, draft, GAMMA, b["token"], b["conf"], b["flag"], b["count"], b["ws"], vocab=V)
    torch.cuda.synchronize()
    tok, conf = b["token"].cpu().numpy(), b["conf"].cpu().numpy()
    _check_rows(tok, conf, ref)
    acc, n = O.verify_accept(rows.draft, tok, conf.astype(np.float64), rows.cu, F32_GAMMA)
    assert np.array_equal(b["flag"].cpu().numpy().astype(bool), acc)
    assert np.array_equal(b["count"].cpu().numpy(), n)
    f2, n2 = torch.full_like(b["flag"], 7), torch.full_like(b["count"], -7)
    dllm.verify_accept(cu, draft, b["token"], b["conf"], GAMMA, f2, n2)
    torch.cuda.synchronize()
    assert torch.equal(f2, b["flag"]) and torch.equal(n2, b["count"])


def test_special_rows(gpu):
    """Constant rows (token 0, confidence 1/V), maxima at the first and the
    last token and on a split boundary, and equal maxima in different splits."""
    import torch
    from io_aware_kv_amd import dllm
    V = 131072
    z = np.zeros((6, V), dtype=np.float32)
    z[1, 0] = 3.0
    z[2, V - 1] = 3.0
    z[3, 8192] = 5.0                         # first token of the second split
    z[4, [8191, 120000]] = 4.0               # twins in different splits
    z[5, :] = -2.5                           # constant, negative
    host = W.round_bf16_bits(z)
    dev = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).to(gpu)
    b = _alloc(6, 1, V, gpu)
    dllm.confidence_argmax(dev, b["token"], b["conf"], b["ws"])
    torch.cuda.synchronize()
    tok, conf = b["token"].cpu().numpy(), b["conf"].cpu().numpy()
    _check_rows(tok, conf, W.bf16_bits_to_f64(host))
    assert tok.tolist() == [0, 0, V - 1, 8192, 8191, 0]
    assert conf[0] == pytest.approx(1.0 / V, rel=1e-4)


def test_decisions_on_given_confidences(gpu):
    """The oracle's hand-worked examples through the standalone entry points."""
    import torch
    from io_aware_kv_amd import dllm
    conf = np.array([0.95, 0.5, 0.9, 0.2, 0.3, 0.6, 0.6, 0.91], dtype=np.float32)
    cu = np.array([0, 4, 7, 7, 8], dtype=np.int32)
    f, n = torch.full((8,), 7, dtype=torch.uint8, device=gpu), torch.full((4,), -7, dtype=torch.int32, device=gpu)
    dllm.confidence_commit(_dev(cu, gpu), _dev(conf, gpu), EPS, f, n)
    torch.cuda.synchronize()
    want, wn = O.confidence_commit(conf.astype(np.float64), cu, F32_EPS)
    assert f.cpu().numpy().astype(bool).tolist() == want.tolist()
    assert n.cpu().numpy().tolist() == wn.tolist() == [2, 1, 0, 1]

    draft = np.array([5, 6, 7, 8, 9, 1, 2, 3], dtype=np.int32)
    pred = np.array([5, 6, 0, 8, 9, 1, 2, 4], dtype=np.int32)
    vconf = np.array([0.9, 0.8, 0.99, 0.99, 0.99, 0.85, 0.79, 0.99], dtype=np.float32)
    cu = np.array([0, 5, 7, 7, 8], dtype=np.int32)
    f.fill_(7)
    n.fill_(-7)
    dllm.verify_accept(_dev(cu, gpu), _dev(draft, gpu), _dev(pred, gpu), _dev(vconf, gpu), GAMMA, f, n)
    torch.cuda.synchronize()
    want, wn = O.verify_accept(draft, pred, vconf.astype(np.float64), cu, F32_GAMMA)
    assert f.cpu().numpy().astype(bool).tolist() == want.tolist()
    assert n.cpu().numpy().tolist() == wn.tolist() == [2, 1, 0, 0]


def test_row_ranges_outside_the_rows_and_long_sequences(gpu):
    """Malformed ranges are clipped to the rows (nothing outside is touched);
    sequences longer than one pass of the decision launch (64 rows) and than
    a workgroup (256 threads) decide like the oracle."""
    import torch
    from io_aware_kv_amd import dllm
    conf = torch.full((8,), 0.95, dtype=torch.float32, device=gpu)
    cu = _dev(np.array([0, 5, 3, 100], dtype=np.int32), gpu)
    f = torch.full((8,), 7, dtype=torch.uint8, device=gpu)
    n = torch.full((3,), -7, dtype=torch.int32, device=gpu)
    dllm.confidence_commit(cu, conf, EPS, f, n)
    torch.cuda.synchronize()
    assert n.cpu().tolist() == [5, 0, 5]       # seq 1 is empty, seq 2 is clipped to rows 3..7
    assert f.cpu().tolist() == [1] * 8

    lens = [5000, 65, 300, 1]
    rows = W.decode_rows(17, lens, 2048, twin_frac=0.2)
    R = int(rows.cu[-1])
    rng = np.random.default_rng(17)
    cf = rng.choice(np.array([0.3, 0.6, 0.85, 0.9, 0.95], dtype=np.float32), size=R)
    cf[:5000] = np.minimum(cf[:5000], np.float32(0.85))          # seq 0: forced decode
    cf[4321] = np.float32(0.89)                                    # its most confident row
    tk = rows.peak_tok.copy()
    cu = _dev(rows.cu, gpu)
    f = torch.full((R,), 7, dtype=torch.uint8, device=gpu)
    n = torch.full((len(lens),), -7, dtype=torch.int32, device=gpu)
    dllm.confidence_commit(cu, _dev(cf, gpu), EPS, f, n)
    torch.cuda.synchronize()
    commit, wn = O.confidence_commit(cf.astype(np.float64), rows.cu, F32_EPS)
    assert np.array_equal(f.cpu().numpy().astype(bool), commit)
    assert np.array_equal(n.cpu().numpy(), wn)
    assert commit[4321] and wn[0] == 1
    vf = np.where(np.arange(R) % 997 == 996, np.float32(0.5), np.float32(0.9)).astype(np.float32)
    f.fill_(7)
    n.fill_(-7)
    dllm.verify_accept(cu, _dev(rows.draft, gpu), _dev(tk, gpu), _dev(vf, gpu), GAMMA, f, n)
    torch.cuda.synchronize()
    acc, an = O.verify_accept(rows.draft, tk, vf.astype(np.float64), rows.cu, F32_GAMMA)
    assert np.array_equal(f.cpu().numpy().astype(bool), acc)
    assert np.array_equal(n.cpu().numpy(), an)


def test_empty_rows(gpu):
    import torch
    from io_aware_kv_amd import dllm
    logits = torch.empty((0, 1000), dtype=torch.bfloat16, device=gpu)
    cu = _dev(np.zeros(3, dtype=np.int32), gpu)
    e32 = torch.empty(0, dtype=torch.int32, device=gpu)
    ef = torch.empty(0, dtype=torch.float32, device=gpu)
    e8 = torch.empty(0, dtype=torch.uint8, device=gpu)
    n = torch.full((2,), -7, dtype=torch.int32, device=gpu)
    dllm.decode_commit(logits, cu, EPS, e32, ef, e8, n, None)
    torch.cuda.synchronize()
    assert n.cpu().tolist() == [0, 0]


def test_full_batch_sampled_rows(gpu):
    """32 sequences x 32 masked window rows at 128 Ki tokens (the batched
    decode shape), device-drawn logits: every row's decision against the
    oracle's rule on the kernel's confidences, and token and confidence of 96
    sampled rows against the oracle."""
    import torch
    from io_aware_kv_amd import dllm
    lens = [32] * 32
    V = W.VOCAB
    rows = W.decode_rows(9, lens, V, twin_frac=0.05)
    dev = W.decode_logits_device(9, rows, V, gpu)
    R = dev.shape[0]
    print(f"[gpu] decode full batch R={R} V={V}", flush=True)
    cu = _dev(rows.cu, gpu)
    b = _alloc(R, len(lens), V, gpu)
    dllm.decode_commit(dev, cu, EPS, b["token"], b["conf"], b["flag"], b["count"], b["ws"])
    torch.cuda.synchronize()
    tok, conf = b["token"].cpu().numpy(), b["conf"].cpu().numpy()
    commit, n = O.confidence_commit(conf.astype(np.float64), rows.cu, F32_EPS)
    assert np.array_equal(b["flag"].cpu().numpy().astype(bool), commit)
    assert np.array_equal(b["count"].cpu().numpy(), n)
    pick = np.sort(np.random.default_rng(2).choice(R, size=96, replace=False))
    ref = dev[torch.from_numpy(pick).to(gpu)].float().cpu().numpy().astype(np.float64)
    _check_rows(tok[pick], conf[pick], ref)
