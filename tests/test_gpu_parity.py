"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element."""
import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import compare, oracle, run_gpu, say, to_np  # noqa: E402

# lengths spanning several 64/128 tiles with ragged tails, one single-token sequence
SELF_LENS = [1, 37, 130, 257]
CROSS_Q = [1, 37, 130, 64]
CROSS_KV = [5, 300, 64, 129]
MODES = [(D, m, a, b) for D in (64, 128) for m in ("none", "causal") for a in ("softmax", "silu", "gelu_tanh")
         for b in ("none", "scalar", "bucket")]


@pytest.mark.parametrize("D,mask,act,bias", MODES, ids=["-".join(map(str, m)) for m in MODES])
def test_tiny_all_modes(D, mask, act, bias):
    lq, lkv = (SELF_LENS, SELF_LENS) if mask == "causal" else (CROSS_Q, CROSS_KV)
    x = ji.make_inputs(lq, lkv, 2, D, wid=40, mask=mask, act=act, bias_kind=bias, bias_sigma=0.5)
    say(f"case tiny D={D} mask={mask} act={act} bias={bias}")
    gpu = run_gpu(x)
    rep = compare(x, gpu, oracle(x))
    say(f"  {rep}")


@pytest.mark.parametrize("act", ["softmax", "silu"])
@pytest.mark.parametrize("slots", [16, 64])
def test_forced_split_matches_oracle_and_unsplit(act, slots):
    lens = [700, 129, 1, 300]
    x = ji.make_inputs(lens, lens, 2, 128, wid=41, mask="causal", act=act, bias_kind="bucket", bias_sigma=0.5)
    say(f"case split act={act} slots={slots}")
    g1 = run_gpu(x, num_slots=slots)
    assert len(g1["plan"].schedule(1)) > 0 and len(g1["plan"].schedule(3)) > 0 and len(g1["plan"].schedule(5)) > 0
    g0 = run_gpu(x, no_split=True)
    assert len(g0["plan"].schedule(1)) == 0
    compare(x, g1, oracle(x))
    # a split piece rounds P to bf16 against its own running max, so the two paths agree to the
    # bf16 operand rounding (unit roundoff 2^-8), not to fp32 rounding
    for name in ["out", "dq", "dk", "dv"]:
        a, b = to_np(g1[name]), to_np(g0[name])
        d = float(np.abs(a - b).max())
        assert d <= 2.0 ** -8 * max(1.0, float(np.abs(b).max())), f"{name}: split vs unsplit differ by {d}"


def test_bf16_outputs():
    lens = [300, 45, 128]
    x = ji.make_inputs(lens, lens, 3, 128, wid=42, mask="causal", act="softmax", bias_kind="bucket")
    say("case bf16 outputs")
    gpu = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    assert gpu["out"].dtype == torch.bfloat16 and gpu["dq"].dtype == torch.bfloat16
    compare(x, gpu, oracle(x), out_bf16=True)


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh"])
def test_empty_sequences(act):
    lq, lkv = [3, 0, 70, 0], [0, 40, 65, 0]
    x = ji.make_inputs(lq, lkv, 2, 64, wid=43, act=act, bias_kind="scalar")
    say(f"case empty act={act}")
    gpu = run_gpu(x)
    ref = oracle(x)
    assert np.all(to_np(gpu["out"])[:3] == 0.0)
    if act == "softmax":
        assert np.all(np.isneginf(to_np(gpu["lse"])[:, :3]))
    assert np.all(to_np(gpu["dq"])[:3] == 0.0) and np.all(to_np(gpu["dk"])[:40] == 0.0)
    compare(x, gpu, ref)


def test_deterministic_and_no_out_of_range_writes():
    lens = [500, 3, 260]
    x = ji.make_inputs(lens, lens, 2, 128, wid=44, mask="causal", bias_kind="bucket")
    say("case determinism + canaries")
    a = run_gpu(x, num_slots=5)
    b = run_gpu(x, num_slots=5)
    for name in ["out", "lse", "dq", "dk", "dv"]:
        assert torch.equal(a[name], b[name]), name
    # canary bands around every output: the kernels must write inside their tensors only
    from jagged_sequence_amd import binding as J
    from tests.gpu_util import to_dev
    plan = a["plan"]
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    qo, ko = torch.from_numpy(x.q_off).cuda(), torch.from_numpy(x.kv_off).cuda()
    bias = torch.from_numpy(x.bias).cuda()
    n = x.q.size
    band = 4096

    def guarded(numel):
        t = torch.full((numel + 2 * band,), 1234.5, dtype=torch.float32, device="cuda")
        return t, t[band:band + numel]

    out_g, out = guarded(n)
    lse_g, lse = guarded(x.H * len(x.q))
    dq_g, dq = guarded(n)
    dk_g, dk = guarded(x.k.size)
    dv_g, dv = guarded(x.v.size)
    out = out.view(x.q.shape)
    plan.forward(q, k, v, qo, ko, bias, out=out, lse=lse.view(x.H, -1))
    plan.backward(q, k, v, qo, ko, bias, out, lse.view(x.H, -1), do, dq=dq.view(x.q.shape), dk=dk.view(x.k.shape),
                  dv=dv.view(x.v.shape))
    torch.cuda.synchronize()
    for g in [out_g, lse_g, dq_g, dk_g, dv_g]:
        assert torch.all(g[:band] == 1234.5) and torch.all(g[-band:] == 1234.5)
    assert torch.equal(out, a["out"]) and torch.equal(dk.view(x.k.shape), a["dk"])


def test_small_workload_forward():
    x = ji.workload_inputs("small_fwd")
    say("case workload small_fwd")
    gpu = run_gpu(x, backward=False)
    rep = compare(x, gpu, oracle(x, backward=False), backward=False)
    gpu16 = run_gpu(x, backward=False, out_dtype="bf16")
    compare(x, gpu16, oracle(x, backward=False), backward=False, out_bf16=True)
    say(f"  {rep}")


def _sample(lq, n_random, seed):
    order = np.argsort(lq)
    rng = np.random.default_rng(seed)
    pick = {int(order[-1]), int(order[0])} | set(rng.choice(len(lq), size=n_random, replace=False).tolist())
    return sorted(pick)


@pytest.mark.parametrize("name", ["causal_bucket", "target_attn", "gdpa_silu", "gdpa_gelu"])
def test_full_size_workloads_sampled(name):
    """Full-size run in the benchmark's launch configuration; the oracle checks sampled sequences."""
    x = ji.workload_inputs(name)
    lq, _ = ji.lengths(ji.WORKLOADS[name])
    seqs = _sample(lq, 3, 7)
    say(f"case workload {name} seqs={seqs}")
    gpu = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    ref = oracle(x, seqs=seqs)
    rep = compare(x, gpu, ref, seqs=seqs, out_bf16=True, plain=True)
    say(f"  {rep}")


# Every sequence with at most 64 queries: softmax dK/dV runs in half-width items (64 keys, 4-wave
# workgroups). Keys span several items with ragged tails.
SHORT_Q = [1, 37, 64, 5]
SHORT_KV = [300, 64, 129, 1000]
SHORT_SELF = [1, 37, 64, 50]


@pytest.mark.parametrize("act", ["softmax", "silu", "gelu_tanh"])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("bias", ["none", "scalar", "bucket"])
def test_short_query_items(mask, bias, act):
    """Every sequence with at most 64 queries: the backward is one fused pass over the dQ items."""
    lq, lkv = (SHORT_SELF, SHORT_SELF) if mask == "causal" else (SHORT_Q, SHORT_KV)
    x = ji.make_inputs(lq, lkv, 2, 128, wid=45, mask=mask, act=act, bias_kind=bias, bias_sigma=0.5)
    say(f"case short-query mask={mask} bias={bias} act={act}")
    gpu = run_gpu(x)
    info = gpu["plan"].info()
    assert info["fused_bwd"] == 1 and info["kv_bn"] == (64 if act == "softmax" else 128)
    compare(x, gpu, oracle(x))


@pytest.mark.parametrize("lq,lkv,fused", [([5, 0, 64, 3], [0, 0, 200, 70], 1), ([0, 30, 64], [50, 40, 129], 0)],
                         ids=["no-keys", "keys-without-queries"])
def test_short_query_empty_sequences(lq, lkv, fused):
    """Short query sets with empty sequences: a sequence without keys (dQ = 0) keeps the fused
    backward; one with keys but no queries (dK = dV = 0 for its keys) takes the separate passes."""
    x = ji.make_inputs(lq, lkv, 2, 128, wid=48, mask="none", act="softmax", bias_kind="bucket", bias_sigma=0.5)
    say(f"case short-query empty sequences lq={lq} lkv={lkv}")
    gpu = run_gpu(x)
    assert gpu["plan"].info()["fused_bwd"] == fused
    compare(x, gpu, oracle(x))


def test_short_query_items_split():
    x = ji.make_inputs(SHORT_Q, SHORT_KV, 2, 128, wid=46, mask="none", act="softmax", bias_kind="bucket",
                       bias_sigma=0.5)
    say("case short-query split")
    g1 = run_gpu(x, num_slots=16)
    # a half-width dK/dV item covers one query tile and is never split; the forward and dQ lists are
    assert g1["plan"].info()["kv_bn"] == 64 and len(g1["plan"].schedule(5)) == 0
    assert len(g1["plan"].schedule(1)) > 0 and len(g1["plan"].schedule(3)) > 0
    compare(x, g1, oracle(x))


# bf16 gradients at D = 128: the dK/dV kernel stages its output rows through LDS on this path.
BF16_GRAD_CASES = [("causal", "softmax", "bucket", False), ("none", "softmax", "scalar", False),
                   ("causal", "silu", "none", False), ("none", "gelu_tanh", "bucket", False),
                   ("none", "softmax", "bucket", True)]


@pytest.mark.parametrize("mask,act,bias,short", BF16_GRAD_CASES, ids=["-".join(map(str, c)) for c in BF16_GRAD_CASES])
def test_bf16_gradients_d128(mask, act, bias, short):
    if short:
        lq, lkv = SHORT_Q, SHORT_KV
    else:
        lq, lkv = (SELF_LENS, SELF_LENS) if mask == "causal" else (CROSS_Q, CROSS_KV)
    x = ji.make_inputs(lq, lkv, 2, 128, wid=47, mask=mask, act=act, bias_kind=bias, bias_sigma=0.5)
    say(f"case bf16 grads mask={mask} act={act} bias={bias} short={short}")
    gpu = run_gpu(x, grad_dtype="bf16")
    assert gpu["dk"].dtype == torch.bfloat16
    assert gpu["plan"].info()["kv_bn"] == (64 if short else 128)
    rep = compare(x, gpu, oracle(x))
    # the same kernels with fp32 gradients: bf16 rounding of each element is the only difference
    g32 = run_gpu(x)
    for name in ["dq", "dk", "dv"]:
        a, b = to_np(gpu[name]), to_np(g32[name])
        assert np.all(np.abs(a - b) <= 2.0 ** -8 * np.abs(b) + 1e-30), name
    say(f"  {rep}")


def _sub_inputs(x, seqs):
    """The listed sequences of a batch as a batch of their own, with their rows in the full layout."""
    import dataclasses
    qr = np.concatenate([np.arange(x.q_off[b], x.q_off[b + 1]) for b in seqs])
    kr = np.concatenate([np.arange(x.kv_off[b], x.kv_off[b + 1]) for b in seqs])
    sub = dataclasses.replace(x, q=x.q[qr], k=x.k[kr], v=x.v[kr], do=None if x.do is None else x.do[qr],
                              q_off=ji.offsets(np.diff(x.q_off)[seqs]), kv_off=ji.offsets(np.diff(x.kv_off)[seqs]))
    return sub, torch.from_numpy(qr).cuda(), torch.from_numpy(kr).cuda()


def _check_longtail_full_size(name):
    """The long-tail workload at full size in the benchmark's launch configuration (bf16 outputs and
    gradients). Whole short sequences go to the oracle. For each 32,768-token sequence the oracle
    evaluates sampled query rows one by one (output, lse, dQ) and the stored oracle values of sampled
    keys give dK / dV element by element (``tests/golden/longtail_keycols.npz``, written by
    ``make_longtail_keycols.py`` from ``oracle.key_cols`` alone); sum_j dK_j = 0 and
    sum_j dV_j = sum_i dO_i per head are checked over every key as well."""
    import os
    from oracle import attention as A
    from tests.gpu_util import LSE_MAX_ABS, OUT_MAX_ABS, rel_l2
    w = ji.WORKLOADS[name]
    x = ji.workload_inputs(name)
    lq, _ = ji.lengths(w)
    short = [int(b) for b in np.argsort(lq, kind="stable")[:1]] + [int(b) for b in np.flatnonzero(lq <= 2048)[[5, 77]]]
    if name == "longtail_1m":
        short += [int(b) for b in np.flatnonzero(lq <= 2048)[[-1]]]  # one of the sequences past the first 512
    longest = [int(b) for b in np.flatnonzero(lq == lq.max())]
    golden = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "longtail_keycols.npz"))
    gseqs = [int(b) for b in golden["seqs"]]
    assert set(gseqs) <= set(longest) and len(gseqs) == 2
    say(f"case workload {name} full size; short seqs {short}, longest {longest}")
    gpu = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    sub, qr, kr = _sub_inputs(x, short)
    g_sub = {"out": gpu["out"][qr], "lse": gpu["lse"][:, qr], "dq": gpu["dq"][qr], "dk": gpu["dk"][kr],
             "dv": gpu["dv"][kr]}
    rep = compare(sub, g_sub, oracle(sub), out_bf16=True, plain=True)
    say(f"  short sequences {rep}")
    f = A.bf16_bits_to_f64
    kw = dict(mask=w.mask, act=w.act, bias_kind=w.bias, bias=x.bias.astype(np.float64))
    for b in longest:
        L = int(lq[b])
        qs, ks = int(x.q_off[b]), int(x.kv_off[b])
        q, k, v, do = (f(t[s:s + L]) for t, s in [(x.q, qs), (x.k, ks), (x.v, ks), (x.do, qs)])
        off = np.array([0, L], dtype=np.int32)
        # Rows drawn uniformly, plus the first and last ones: the sample's rel-L2 of dQ estimates that of
        # the whole sequence, which is what the gradient bound is stated for. (A row with two visible
        # keys alone can be off by several percent: Delta = dO . O uses the stored bf16 output and
        # dP - Delta cancels there; whole short sequences, which contain such rows, are checked above.)
        rng = np.random.default_rng(b)
        sel = sorted({0, 1, 2, L - 1} | set(rng.choice(L, 60, replace=False).tolist()))
        uniform = [r for r, i in enumerate(sel) if i not in (1, 2)]
        rows = [qs + i for i in sel]
        for h in (0, w.H - 1):
            o, l, g = A.rows(q, k, v, off, off, 0, h, sel, do, **kw)
            og = gpu["out"][rows, h].float().cpu().numpy().astype(np.float64)
            lg = gpu["lse"][h, rows].cpu().numpy().astype(np.float64)
            gg = gpu["dq"][rows, h].float().cpu().numpy().astype(np.float64)
            bound = OUT_MAX_ABS + np.exp2(np.floor(np.log2(np.maximum(np.abs(o), 1e-30))) - 8)
            assert np.all(np.abs(og - o) <= bound), (b, h, np.abs(og - o).max())
            assert np.abs(lg - l).max() <= LSE_MAX_ABS, (b, h, np.abs(lg - l).max())
            err = rel_l2(gg[uniform], g[uniform])
            assert err <= 2e-2, (b, h, err)
            msg = (f"  seq {b} head {h}: out max-abs {np.abs(og - o).max():.2e}, lse {np.abs(lg - l).max():.2e}, "
                   f"dQ rel-L2 (sampled rows) {err:.2e}")
            if b in gseqs:
                keys = golden[f"keys_{b}"]
                dkg = gpu["dk"][ks + torch.from_numpy(keys).cuda(), h].double().cpu().numpy()
                dvg = gpu["dv"][ks + torch.from_numpy(keys).cuda(), h].double().cpu().numpy()
                ek = rel_l2(dkg, golden[f"dk_{b}_{h}"].astype(np.float64))
                ev = rel_l2(dvg, golden[f"dv_{b}_{h}"].astype(np.float64))
                first = keys < 128
                ek0 = rel_l2(dkg[first], golden[f"dk_{b}_{h}"][first].astype(np.float64))
                assert ek <= 2e-2 and ev <= 2e-2 and ek0 <= 2e-2, (b, h, ek, ev, ek0)
                msg += f", dK / dV rel-L2 (sampled keys) {ek:.2e} / {ev:.2e}, first key tile dK {ek0:.2e}"
            say(msg)
        dk = gpu["dk"][ks:ks + L].double()
        dv = gpu["dv"][ks:ks + L].double()
        dO = torch.from_numpy(do).to(dk.device)
        for hh in range(w.H):
            s_dk = dk[:, hh].sum(0).norm().item()
            assert s_dk <= 1e-3 * dk[:, hh].norm(dim=1).sum().item(), (b, hh, s_dk)
            err = (dv[:, hh].sum(0) - dO[:, hh].sum(0)).norm().item()
            assert err <= 1e-2 * dO[:, hh].sum(0).norm().item(), (b, hh, err)
    say("  longest sequences: sampled rows, sampled keys and gradient identities within bounds")


def test_full_size_longtail_max_length():
    """Long-tail workload, B = 512 (333,877 tokens)."""
    _check_longtail_full_size("longtail")


def test_full_size_longtail_1m():
    """Long-tail workload at about a million tokens (B = 1652, 1,000,301 tokens, four 32,768-token
    sequences)."""
    _check_longtail_full_size("longtail_1m")
