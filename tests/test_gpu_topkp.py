"""GPU parity of spec_verify_topkp (top-k / top-p truncation before the
verify step) against the oracle, through the C ABI.

Each request gets its own (top_k, top_p) from a mix that covers truncation
off, top-k alone (1, small, large, V - 1, beyond V, negative), top-p alone
(0.3 to 0.999999) and both together. Inputs: ragged bf16 and fp32 batches
at several temperatures (greedy included), the full-vocabulary workload
(every request run on the GPU, a sample checked against the oracle),
logits on a coarse grid so that top-k and top-p cut through runs of equal
values, rows holding -inf, and bad top_p values.

Which prefix top-p keeps is decided by floating point. The kernel forms
each token's weight e^(s - max s) to within about 2.4e-7 relative (the
exponent split exactly, one v_exp_f32 of at most 1 ulp, two binary32
roundings) and sums the weights exactly in fixed point, so its cumulative
weight and the top-p target are each within 2.4e-7 of the kept total: its
decision can differ from the exact one only where the oracle's decision
margin (``trunc_margin``, relative to the kept total) is below 4.8e-7. Such
requests are excused and counted (their outputs must still be well formed);
every other request must meet the verify parity rules."""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth
from oracle import verify as ov

from .gpu_util import announce, device, run_verify, verify_inputs
from .parity import check_excused_bound, compare_verify

pytestmark = pytest.mark.gpu

TRUNC_MARGIN = 5e-7


def _settings(B, V, rotate=0):
    mix = [(0, 1.0), (1, 1.0), (5, 1.0), (50, 1.0), (1000, 1.0), (V - 1, 1.0), (V + 3, 1.0),
           (-1, 0.3), (0, 0.5), (0, 0.9), (0, 0.95), (0, 0.999), (7, 0.999999), (20, 0.8),
           (3000, 0.95), (100000, 0.9), (2, 0.6)]
    mix = mix[rotate % len(mix):] + mix[:rotate % len(mix)]
    top_k = np.array([mix[b % len(mix)][0] for b in range(B)], dtype=np.int32)
    top_p = np.array([mix[b % len(mix)][1] for b in range(B)], dtype=np.float32)
    return top_k, top_p


def _run_gpu(case, top_k, top_p, dev):
    inp = verify_inputs(case, dev)
    acc, toks, alpha, status = lv.spec_verify_topkp(
        **inp, top_k=torch.from_numpy(top_k).to(dev), top_p=torch.from_numpy(top_p).to(dev))
    torch.cuda.synchronize(dev)
    return {"accepted_len": acc.cpu().numpy(), "tokens": toks.cpu().numpy(),
            "alpha": alpha.cpu().numpy(), "status": status.cpu().numpy()}


def _oracle(case, top_k, top_p, requests):
    kmax = case.draft.shape[1]
    res = [ov.verify_request(ov.decode_rows(case.target[b], case.dtype),
                             ov.decode_rows(case.draft[b], case.dtype), case.tokens[b],
                             case.k[b], case.temperature[b], int(case.seed[b]), b, kmax,
                             top_k=int(top_k[b]), top_p=float(top_p[b]))
           for b in requests]
    keys = ("accepted_len", "tokens", "alpha", "accept_margin", "draw_margin", "status",
            "greedy", "trunc_margin")
    return {k: np.array([r[k] for r in res]) for k in keys}


def _compare(case, gpu, top_k, top_p, tag, requests=None):
    B = case.shape[0]
    requests = list(range(B)) if requests is None else list(requests)
    orc = _oracle(case, top_k, top_p, requests)
    keep = [i for i, _ in enumerate(requests) if not orc["trunc_margin"][i] < TRUNC_MARGIN]
    excused = len(requests) - len(keep)
    V = case.shape[2]
    for i, b in enumerate(requests):
        if i in keep:
            continue
        # an excused request: same status, well-formed outputs
        assert gpu["status"][b] == orc["status"][i], (tag, b)
        j, kb = int(gpu["accepted_len"][b]), int(case.k[b])
        assert 0 <= j <= kb, (tag, b)
        t = gpu["tokens"][b]
        assert np.array_equal(t[:j], case.tokens[b][:j]) and 0 <= t[j] < V \
            and np.all(t[j + 1:] == -1), (tag, b)
        assert np.all((gpu["alpha"][b][:kb] >= 0) & (gpu["alpha"][b][:kb] <= 1 + 1e-6)), (tag, b)
    sel = [requests[i] for i in keep]
    g = {k: v[sel] for k, v in gpu.items()}
    o = {k: v[keep] for k, v in orc.items()}
    rep = compare_verify(g, o, case.k[sel], case.shape[1])
    announce(f"topkp {tag}: {len(requests)} requests, {rep['stochastic']} stochastic, "
             f"{rep['greedy']} greedy, {rep['faulted']} faulted, truncation near-ties "
             f"excused {excused}, accept {rep['excused_accept']}, draw {rep['excused_draw']}")
    assert not rep["failures"], (tag, [(sel[i], why) for i, why in rep["failures"][:5]])
    check_excused_bound(rep, tag)
    # Truncation near-ties are not bounded: the settings include top-p 0.999
    # and 0.999999, whose decision falls among tail tokens each holding about
    # 1e-7 of the kept weight, so small margins are what those rows are for.
    # How many of the excused requests actually differ is reported.
    differ = sum(1 for i, b in enumerate(requests) if i not in keep and not (
        gpu["accepted_len"][b] == orc["accepted_len"][i] and
        np.array_equal(gpu["tokens"][b], orc["tokens"][i])))
    announce(f"topkp {tag}: truncation near-tie requests that differ from the oracle: {differ}")
    return rep, excused


@pytest.mark.parametrize("dtype_case,temperature", [(3, 1.0), (3, 0.6), (3, 1.7), (1, 1.0)])
def test_topkp_ragged_against_oracle(dtype_case, temperature):
    dev = device()
    if dtype_case == 3:
        case = synth.verify_case(3, temperature=temperature, batch=34, vocab=9001,
                                 k_values=[(b * 5) % 8 for b in range(34)])
    else:
        case = synth.verify_case(1, temperature=temperature, batch=17, vocab=4096, kmax=4)
    top_k, top_p = _settings(case.shape[0], case.shape[2], rotate=int(temperature * 10))
    announce(f"topkp ragged case={dtype_case} T={temperature} shape={case.shape}")
    _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p,
             f"ragged case={dtype_case} T={temperature}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("temperature", [0.7, 1.3])
def test_topp_wide_cuts_against_oracle(dtype, temperature):
    """Top-p cuts in the body of Zipf-shaped rows, aligned rows of both
    dtypes, against the oracle. At T = 1.3 the rows are flat enough that the
    cuts keep more tokens than the selection list holds, so the row kernel
    makes its one pass with the keep rule on the raw logits (bounds found by
    bisection over the input format, T != 1); at T = 0.7 they keep a few
    hundred and take the list path."""
    dev = device()
    case = synth.verify_case(3, temperature=temperature, batch=12, vocab=24576,
                             k_values=[(b * 3) % 8 for b in range(12)])
    if dtype == "f32":
        case.dtype = "f32"
        case.target = synth.from_bf16(case.target)
        case.draft = synth.from_bf16(case.draft)
    B = case.shape[0]
    top_k = np.zeros(B, np.int32)
    # cuts in the body of the distribution, where the boundary token's own
    # weight keeps the truncation margin above the excusal threshold
    top_p = np.array([0.9, 0.95, 0.8, 0.97, 0.85, 0.93] * 2, np.float32)[:B]
    announce(f"topp wide cuts {dtype} T={temperature} shape={case.shape}")
    _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p,
             f"wide cuts {dtype} T={temperature}")


def test_topkp_greedy_and_mixed_temperatures():
    dev = device()
    case = synth.verify_case(3, batch=17, vocab=5000, kmax=5)
    case.temperature[:] = np.array([0.0, 1.0, 0.5, 2.0] * 5, dtype=np.float32)[:17]
    case = synth.redraw_tokens(case, 1.0)
    case.temperature[:] = np.array([0.0, 1.0, 0.5, 2.0] * 5, dtype=np.float32)[:17]
    top_k, top_p = _settings(17, 5000, rotate=3)
    announce(f"topkp mixed temperatures shape={case.shape}")
    rep, _ = _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p, "mixed T")
    assert rep["greedy"] >= 4


def _grid_case(dtype, step, V=6000, B=17, K=3, with_ninf=False):
    """Logits on a grid of `step` (many exact ties), in `dtype`."""
    rng = np.random.default_rng(int(step * 100) + (dtype == "bf16"))
    t = np.round(rng.standard_normal((B, K + 1, V)) * 2.0 / step) * step
    d = np.round((t[:, :K] + 0.7 * rng.standard_normal((B, K, V))) / step) * step
    t = t.astype(np.float32)
    d = d.astype(np.float32)
    if with_ninf:
        t[:, :, ::7] = -np.inf
        d[:, :, 3::11] = -np.inf
    case = synth.verify_case(1, batch=B, vocab=V, kmax=K)
    case.dtype = dtype
    case.target = synth.to_bf16(t) if dtype == "bf16" else t
    case.draft = synth.to_bf16(d) if dtype == "bf16" else d
    dec = ov.decode_rows(case.draft.reshape(-1, V), dtype).reshape(B, K, V)
    case.tokens = np.argmax(dec + rng.gumbel(size=dec.shape), axis=-1).astype(np.int32)
    case.k = np.full(B, K, dtype=np.int32)
    case.temperature = np.full(B, 1.0, dtype=np.float32)
    case.seed = rng.integers(0, 2**63, size=B).astype(np.uint64)
    return case


@pytest.mark.parametrize("dtype,step,ninf", [("bf16", 0.25, False), ("f32", 0.5, False),
                                             ("f32", 0.125, True), ("bf16", 1.0, True)])
def test_topkp_cuts_through_equal_logits(dtype, step, ninf):
    dev = device()
    case = _grid_case(dtype, step, with_ninf=ninf)
    B, _, V = case.shape
    top_k, top_p = _settings(B, V, rotate=5)
    top_k[::3] = [3, 17, 250, 999, 4000, 31][:len(top_k[::3])]
    announce(f"topkp ties dtype={dtype} step={step} -inf={ninf} shape={case.shape}")
    _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p,
             f"ties {dtype} step={step} ninf={ninf}")


def test_topkp_constant_rows_keep_lowest_ids():
    """All logits equal: top-k keeps ids 0..k-1, top-p the shortest prefix of
    ids; with k = 1 every draw is token 0."""
    dev = device()
    B, K, V = 6, 2, 1000
    case = synth.verify_case(1, batch=B, vocab=V, kmax=K)
    case.target = np.zeros((B, K + 1, V), np.float32)
    case.draft = np.zeros((B, K, V), np.float32)
    case.tokens = np.array([[0, 1], [5, 0], [0, 0], [999, 3], [2, 2], [0, 9]], np.int32)
    case.k = np.full(B, K, np.int32)
    case.temperature = np.ones(B, np.float32)
    case.seed = np.arange(B, dtype=np.uint64) * 7919
    top_k = np.array([1, 10, 1, 0, 3, 0], np.int32)
    top_p = np.array([1.0, 1.0, 0.5, 0.0105, 1.0, 0.3517], np.float32)
    announce("topkp constant rows")
    gpu = _run_gpu(case, top_k, top_p, dev)
    _compare(case, gpu, top_k, top_p, "constant rows")
    for b in (0, 2):   # k = 1 keeps token 0 only: the draw is 0
        j = gpu["accepted_len"][b]
        assert gpu["tokens"][b][j] == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topkp_crowded_bins(dtype):
    """Rows of a few distinct logits with V = 30000: the bin holding the
    top-k or top-p boundary has more tokens than one workgroup gathers, so
    the selection refines it by passes over the row instead."""
    dev = device()
    B, K, V = 8, 2, 30000
    rng = np.random.default_rng(17 if dtype == "bf16" else 18)
    vals = np.array([1.0, 0.5, 0.0, -3.0], np.float32)
    t = vals[rng.integers(0, 4, (B, K + 1, V))]
    d = vals[rng.integers(0, 4, (B, K, V))]
    t[:, :, 123] = 2.0           # one clear maximum per row
    case = synth.verify_case(1, batch=B, vocab=V, kmax=K)
    case.dtype = dtype
    case.target = synth.to_bf16(t) if dtype == "bf16" else t
    case.draft = synth.to_bf16(d) if dtype == "bf16" else d
    case.tokens = rng.integers(0, V, (B, K)).astype(np.int32)
    case.k = np.full(B, K, np.int32)
    case.temperature = np.array([1.0, 0.7, 1.0, 1.3, 1.0, 1.0, 0.9, 1.0], np.float32)
    case.seed = rng.integers(0, 2**63, size=B).astype(np.uint64)
    top_k = np.array([9000, 20000, 0, 0, 15000, 29999, 1, 12000], np.int32)
    top_p = np.array([1.0, 1.0, 0.4, 0.77, 0.6, 0.3, 1.0, 0.93], np.float32)
    announce(f"topkp crowded bins dtype={dtype} shape={case.shape}")
    _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p, f"crowded {dtype}")


@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_topkp_first_tile_holds_the_top_tokens(temperature):
    """Most of the top-50 tokens sit in the row's first 4096 ids, so the
    list the selection's first pass builds from the first tile's counts
    stops above the 50th token and a second pass gathers the boundary;
    other rows push that list past its capacity. Checked against the
    oracle."""
    dev = device()
    B, K, V = 6, 2, 100000
    rng = np.random.default_rng(61)
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + 0.5 * rng.standard_normal((B, K, V))).astype(np.float32)
    for b in range(B):
        for rows in (t[b], d[b]):
            if b % 2 == 0:      # 40 high tokens in the first tile, 30 a little lower elsewhere
                rows[:, rng.choice(4096, 40, replace=False)] = 6.0 + rng.random((rows.shape[0], 40))
                rows[:, 4096 + rng.choice(V - 4096, 30, replace=False)] = 5.0 + rng.random((rows.shape[0], 30))
            else:               # a few very high tokens in the first tile, its other tokens very low
                rows[:, :4096] = -20.0
                rows[:, rng.choice(4096, 30, replace=False)] = 10.0 + rng.random((rows.shape[0], 30))
    case = synth.verify_case(1, batch=B, vocab=V, kmax=K)
    case.dtype = "bf16"
    case.target = synth.to_bf16(t)
    case.draft = synth.to_bf16(d)
    dec = ov.decode_rows(case.draft.reshape(-1, V), "bf16").reshape(B, K, V)
    case.tokens = np.argmax(dec / temperature + rng.gumbel(size=dec.shape), axis=-1).astype(np.int32)
    case.k = np.full(B, K, np.int32)
    case.temperature = np.full(B, temperature, np.float32)
    case.seed = rng.integers(0, 2**63, size=B).astype(np.uint64)
    top_k = np.array([50, 50, 45, 60, 50, 35], np.int32)
    top_p = np.array([1.0, 0.9, 0.95, 1.0, 0.8, 0.99], np.float32)
    announce(f"topkp first tile heavy T={temperature} shape={case.shape}")
    _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p, f"first tile T={temperature}")


def test_bad_top_p_faults_with_other_bits():
    dev = device()
    case = synth.verify_case(3, batch=6, vocab=3000, kmax=2)
    case.temperature[3] = -1.0            # also a bad temperature
    case.tokens[4, 0] = 3000              # also a bad token
    top_k = np.zeros(6, np.int32)
    top_p = np.array([0.0, -0.5, np.nan, 0.0, 0.0, 0.9], np.float32)
    announce("topkp bad top_p")
    gpu = _run_gpu(case, top_k, top_p, dev)
    orc = _oracle(case, top_k, top_p, range(6))
    assert list(gpu["status"]) == list(orc["status"])
    assert gpu["status"][0] == lv.STATUS_BAD_TRUNCATION
    assert gpu["status"][3] == lv.STATUS_BAD_TRUNCATION | lv.STATUS_BAD_TEMPERATURE
    assert gpu["status"][4] == lv.STATUS_BAD_TRUNCATION | lv.STATUS_BAD_TOKEN
    assert gpu["status"][5] == 0
    assert np.all(gpu["accepted_len"][:5] == -1)


def test_topkp_workspace_contents_do_not_matter():
    """The kept prefixes, the kept-token lists and their lengths in the
    workspace are written before they are read: a workspace full of garbage
    gives the same outputs as a fresh one, and so does one that an earlier
    call with other settings left behind."""
    dev = device()
    case = synth.verify_case(3, temperature=0.8, batch=12, vocab=40000)
    B, kmax, V = case.shape
    top_k, top_p = _settings(B, V, rotate=2)
    nbytes = lv.spec_verify_topkp_workspace_bytes(B, kmax, V, lv.LVTV_BF16)
    fresh = lv.new_workspace(nbytes, dev)
    junk = lv.new_workspace(nbytes, dev)
    junk.fill_(0xA7)
    used = lv.new_workspace(nbytes, dev)
    inp = verify_inputs(case, dev)
    tk = torch.from_numpy(top_k).to(dev)
    tp = torch.from_numpy(top_p).to(dev)
    # an earlier call on `used` with every request truncated to top-k 3
    lv.spec_verify_topkp(**inp, top_k=torch.full_like(tk, 3), top_p=torch.ones_like(tp),
                         workspace=used)
    announce(f"topkp workspace garbage shape={case.shape}")
    outs = []
    for ws in (fresh, junk, used):
        acc, toks, alpha, status = lv.spec_verify_topkp(**inp, top_k=tk, top_p=tp, workspace=ws)
        torch.cuda.synchronize(dev)
        outs.append((acc.cpu().numpy(), toks.cpu().numpy(), alpha.cpu().numpy(),
                     status.cpu().numpy()))
    for other in outs[1:]:
        for x, y in zip(outs[0], other):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("vocab", [600000, 600001])
def test_topkp_large_vocabulary(vocab):
    """Rows of more than 1024 chunks (V > 524288): the row kernel keeps no
    list of kept tokens and applies the keep rule to the whole row."""
    dev = device()
    case = synth.verify_case(3, temperature=1.0, batch=6, vocab=vocab, kmax=2)
    B, _, V = case.shape
    top_k = np.array([50, 0, 1000, 5, 0, 200000], np.int32)
    top_p = np.array([0.9, 0.8, 1.0, 1.0, 0.95, 0.5], np.float32)
    announce(f"topkp large vocabulary shape={case.shape}")
    _compare(case, _run_gpu(case, top_k, top_p, dev), top_k, top_p, f"V={vocab}")


def _offset_copy(t, offset):
    """The values of `t` stored `offset` elements past a fresh allocation's
    start: rows whose base is not 16-byte aligned."""
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=t.device)
    view = flat[offset:].view(t.shape)
    view.copy_(t)
    return view


@pytest.mark.parametrize("temperature", [0.7, 1.0])
def test_topkp_unaligned_rows_match_aligned(temperature):
    """Rows that are not 16-byte aligned (offset copies of the inputs) take
    the unaligned loads in the selection and the row kernel; outputs must be
    bit-identical to those of the aligned inputs."""
    dev = device()
    case = synth.verify_case(3, temperature=temperature, batch=17, vocab=40000)
    B, _, V = case.shape
    top_k, top_p = _settings(B, V, rotate=4)
    inp = verify_inputs(case, dev)
    tk = torch.from_numpy(top_k).to(dev)
    tp = torch.from_numpy(top_p).to(dev)
    shifted = dict(inp)
    shifted["target_logits"] = _offset_copy(inp["target_logits"], 1)
    shifted["draft_logits"] = _offset_copy(inp["draft_logits"], 3)
    announce(f"topkp unaligned rows T={temperature} shape={case.shape}")
    outs = []
    for x in (inp, shifted):
        acc, toks, alpha, status = lv.spec_verify_topkp(**x, top_k=tk, top_p=tp)
        torch.cuda.synchronize(dev)
        outs.append((acc.cpu().numpy(), toks.cpu().numpy(), alpha.cpu().numpy().view(np.uint32),
                     status.cpu().numpy()))
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("vocab", [None, 30000])
def test_truncation_off_equals_plain_verify(vocab):
    """top_k <= 0 or >= V and top_p >= 1 keep every token: the outputs are
    bit-identical to spec_verify's, on the full-vocabulary workload and on
    short rows (7 tiles and a partial one)."""
    dev = device()
    case = synth.verify_case(3, temperature=0.6, batch=16, vocab=vocab)
    B, _, V = case.shape
    top_k = np.where(np.arange(B) % 2 == 0, 0, V).astype(np.int32)
    top_p = np.where(np.arange(B) % 3 == 0, 1.0, 2.5).astype(np.float32)
    announce(f"topkp off vs plain shape={case.shape}")
    plain = run_verify(case, dev)
    trunc = _run_gpu(case, top_k, top_p, dev)
    for key in ("accepted_len", "status", "tokens", "alpha"):
        assert np.array_equal(plain[key], trunc[key]), key


def test_topkp_full_vocabulary_workload():
    """The full batch (B = 64, Kmax = 7, V = 151936, bf16) on the GPU in one
    call; 16 requests spread over the batch checked against the oracle."""
    dev = device()
    case = synth.verify_case(3)
    B, _, V = case.shape
    top_k, top_p = _settings(B, V)
    announce(f"topkp full workload shape={case.shape}")
    gpu = _run_gpu(case, top_k, top_p, dev)
    sample = list(range(0, B, 4))
    _compare(case, gpu, top_k, top_p, "full workload (sample)", requests=sample)
    # a rerun is bit-identical
    again = _run_gpu(case, top_k, top_p, dev)
    for key in ("accepted_len", "tokens", "alpha", "status"):
        assert np.array_equal(gpu[key], again[key]), key
