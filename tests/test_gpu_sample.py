"""Speculative sampling on the device (gdn_spec_accept_sample) against the
oracle (oracle/sampling.py), through the C ABI.

accept_len and next_token are integers decided by floating point: the device
forms p, q and the Gumbel keys in fp32, the oracle in fp64 on the same
(bf16-rounded) logits and the same Philox words. They must agree bit for bit
wherever the oracle's decision is clear of a tie; a request whose acceptance
comparison is within 1e-4 (relative) of equality, or whose two best keys are
within 1e-3, is only checked for validity (an accept length in range, a token
of the vocabulary), and the seeded cases hold few such requests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
import parity as par  # noqa: E402
from oracle import sampling as smp  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"
ACCEPT_TIE = 1e-4
KEY_TIE = 1e-3


def _softmax(x):
    z = np.exp(x - x.max(-1, keepdims=True))
    return z / z.sum(-1, keepdims=True)


def make_inputs(B, R, V, seed, dtype="bf16", probs=True, penalties=True, pad=(), scale=2.0):
    """Seeded logits ~ N(0, scale^2); drafts drawn from a drafter distribution
    q = softmax(logits of the row + noise) (or its argmax for a greedy
    drafter); prior counts mostly zero."""
    rng = np.random.default_rng(seed)
    logits = (scale * rng.standard_normal((B, R, V))).astype(np.float32)
    if dtype == "bf16":
        logits = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(logits))
    q = _softmax(logits[:, :max(R - 1, 0)].astype(np.float64) + rng.standard_normal((B, max(R - 1, 0), V)))
    q = q.astype(np.float32)
    if probs:
        draft = np.array([[rng.choice(V, p=q[b, t] / q[b, t].sum()) for t in range(R - 1)] for b in range(B)],
                         np.int32).reshape(B, R - 1)
    else:
        draft = q.argmax(-1).astype(np.int32).reshape(B, R - 1)
        flip = rng.random((B, R - 1)) < 0.3
        draft = np.where(flip, rng.integers(0, V, (B, R - 1)), draft).astype(np.int32)
    d = {"logits": logits, "draft": draft, "draft_probs": q if probs else None,
         "temperature": rng.uniform(0.5, 1.5, B).astype(np.float32),
         "slot_ids": np.where(np.isin(np.arange(B), pad), -1, np.arange(B)).astype(np.int32)}
    if penalties:
        d["pending"] = rng.integers(0, V, B).astype(np.int32)
        d["prior_counts"] = np.where(rng.random((B, V)) < 0.9, 0, rng.integers(1, 4, (B, V))).astype(np.int32)
        d["presence"] = rng.uniform(0.0, 1.0, B).astype(np.float32)
        d["frequency"] = rng.uniform(0.0, 0.5, B).astype(np.float32)
    return d


def run_device(d, seed, dtype="bf16"):
    B, R, V = d["logits"].shape
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    lg = torch.from_numpy(d["logits"]).to(DEV)
    lg = lg.to(torch.bfloat16) if dtype == "bf16" else lg   # exact: the values are bf16 already
    acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scratch = torch.empty(bd.gdn_spec_sample_scratch_bytes(B, R, V), dtype=torch.uint8, device=DEV)
    bd.gdn_spec_accept_sample(lg, t(d["draft"]), t(d["temperature"]), seed, acc, nxt, scratch,
                              draft_probs=t(d.get("draft_probs")), pending=t(d.get("pending")),
                              prior_counts=t(d.get("prior_counts")), presence=t(d.get("presence")),
                              frequency=t(d.get("frequency")), slot_ids=t(d.get("slot_ids")), err_flag=err)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), int(err.item())


def run_oracle(d, seed):
    return smp.speculative_sample(d["logits"], d["draft"], seed, d["temperature"], draft_probs=d.get("draft_probs"),
                                  pending=d.get("pending"), prior_counts=d.get("prior_counts"),
                                  presence=d.get("presence"), frequency=d.get("frequency"),
                                  slot_ids=d.get("slot_ids"), details=True)


def compare(d, seed, dtype):
    acc, nxt, err = run_device(d, seed, dtype)
    acc_r, nxt_r, info = run_oracle(d, seed)
    assert err == 0
    B, R, V = d["logits"].shape
    ties = 0
    for b in range(B):
        i = info[b]
        if i is None:            # padding
            assert acc[b] == 0 and nxt[b] == -1
            continue
        clear = min(i["accept_margins"][:acc_r[b]] or [1.0]) > ACCEPT_TIE and i["argmax_gap"] > KEY_TIE
        if clear:
            assert acc[b] == acc_r[b] and nxt[b] == nxt_r[b], (b, acc[b], acc_r[b], nxt[b], nxt_r[b], i)
        else:
            ties += 1
            assert 1 <= acc[b] <= R and 0 <= nxt[b] < V
    assert ties <= max(1, B // 20), ties
    return acc_r


CASES = [
    # B, R, V, dtype, draft probabilities, penalties, padding
    (16, 4, 1000, "f32", False, False, ()),
    (16, 9, 5000, "bf16", True, True, (3, 11)),
    (24, 3, 4097, "bf16", True, False, ()),          # one entry past a whole split
    (8, 9, 3, "f32", True, True, ()),                # vocabulary smaller than a unit
    (32, 5, 20000, "bf16", False, True, (0,)),
]


@pytest.mark.parametrize("B,R,V,dtype,probs,pen,pad", CASES)
def test_sample_matches_oracle(B, R, V, dtype, probs, pen, pad):
    print("sample B=%d R=%d V=%d %s probs=%d pen=%d" % (B, R, V, dtype, probs, pen), flush=True)
    d = make_inputs(B, R, V, seed=B * 1000 + V, dtype=dtype, probs=probs, penalties=pen, pad=pad)
    for seed in (12345, 2**40 + 77):
        compare(d, seed, dtype)


def test_sample_full_vocabulary():
    """A Qwen-sized vocabulary (151936 entries: 38 splits, the last one
    ragged), bonus draws only (R = 1) and 9 rows with a greedy drafter."""
    for R in (1, 9):
        print("sample full vocabulary R=%d" % R, flush=True)
        d = make_inputs(6, R, 151936, seed=R, dtype="bf16", probs=False, penalties=True)
        compare(d, 99 + R, "bf16")


def test_sample_accept_length_spread():
    """The seeded drafter agrees with the target often enough that every
    accept length from 1 to R occurs: the run stops at every row."""
    d = make_inputs(64, 4, 64, seed=5, dtype="f32", probs=True, penalties=False, scale=0.5)
    acc_r = compare(d, 777, "f32")
    assert set(acc_r.tolist()) == {1, 2, 3, 4}


def test_scratch_reused_across_calls():
    """One scratch buffer for several calls in a row (the call resets its own
    counters): a full batch, then a smaller one with another vocabulary, then
    the first again with a new seed; each against the oracle."""
    big = make_inputs(24, 9, 30000, seed=77, dtype="bf16", probs=False, penalties=True)
    small = make_inputs(5, 4, 4500, seed=78, dtype="f32", probs=True, penalties=False)
    nbytes = max(bd.gdn_spec_sample_scratch_bytes(24, 9, 30000), bd.gdn_spec_sample_scratch_bytes(5, 4, 4500))
    scratch = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=DEV)   # not cleared: garbage to start
    for d, seed, dtype in ((big, 11, "bf16"), (small, 12, "f32"), (big, 13, "bf16")):
        B, R, V = d["logits"].shape
        print("sample reuse B=%d R=%d V=%d seed=%d" % (B, R, V, seed), flush=True)
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        lg = torch.from_numpy(d["logits"]).to(DEV)
        lg = lg.to(torch.bfloat16) if dtype == "bf16" else lg
        acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        bd.gdn_spec_accept_sample(lg, t(d["draft"]), t(d["temperature"]), seed, acc, nxt, scratch,
                                  draft_probs=t(d.get("draft_probs")), pending=t(d.get("pending")),
                                  prior_counts=t(d.get("prior_counts")), presence=t(d.get("presence")),
                                  frequency=t(d.get("frequency")), slot_ids=t(d.get("slot_ids")), err_flag=err)
        torch.cuda.synchronize()
        acc_r, nxt_r, info = run_oracle(d, seed)
        assert int(err.item()) == 0
        clear = [min(i["accept_margins"][:acc_r[b]] or [1.0]) > ACCEPT_TIE and i["argmax_gap"] > KEY_TIE
                 for b, i in enumerate(info)]
        a, n = acc.cpu().numpy(), nxt.cpu().numpy()
        assert all((a[b] == acc_r[b] and n[b] == nxt_r[b]) or not clear[b] for b in range(B)), (a, acc_r, n, nxt_r)
        assert sum(not c for c in clear) <= max(1, B // 20)


def test_bad_inputs_are_flagged():
    d = make_inputs(6, 4, 100, seed=9, dtype="f32", probs=False, penalties=True)
    d["temperature"][1] = 0.0
    d["temperature"][2] = np.nan
    d["draft"][3, 1] = 100          # outside the vocabulary
    d["pending"][4] = -1
    acc, nxt, err = run_device(d, 3, "f32")
    assert err == 8
    for b in (1, 2, 3, 4):
        assert acc[b] == 0 and nxt[b] == -1
    assert 1 <= acc[0] <= 4 and 1 <= acc[5] <= 4


def test_verify_sample_commit_chain():
    """verify -> speculative sampling -> commit, the accept lengths never
    leaving the device: the committed state and history equal the oracle's
    for the oracle's accept lengths (which the device reproduced)."""
    w = wl.WORKLOADS["low-concurrency"]
    sid, _ = wl.draw_requests(w)
    sid[3] = -1
    c = gh.make_case(w, slot_ids=sid)
    V = 2048
    d = make_inputs(w.batch, w.rows, V, seed=21, dtype="bf16", probs=True, penalties=True)
    d["slot_ids"] = sid
    acc_r, nxt_r, info = run_oracle(d, 4242)
    assert all(i is None or (min(i["accept_margins"][:acc_r[b]] or [1.0]) > ACCEPT_TIE and i["argmax_gap"] > KEY_TIE)
               for b, i in enumerate(info)), "the seeded chain case should hold no near-ties"
    gh.verify(c)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    nxt = torch.empty(w.batch, dtype=torch.int32, device=DEV)
    scratch = torch.empty(bd.gdn_spec_sample_scratch_bytes(w.batch, w.rows, V), dtype=torch.uint8, device=DEV)
    bd.gdn_spec_accept_sample(torch.from_numpy(d["logits"]).to(DEV).to(torch.bfloat16), t(d["draft"]),
                              t(d["temperature"]), 4242, c.accept, nxt, scratch, draft_probs=t(d["draft_probs"]),
                              pending=t(d["pending"]), prior_counts=t(d["prior_counts"]), presence=t(d["presence"]),
                              frequency=t(d["frequency"]), slot_ids=c.slot_ids)
    gh.commit(c)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
    assert np.array_equal(c.accept.cpu().numpy(), acc_r)
    assert np.array_equal(nxt.cpu().numpy(), nxt_r)
    ref = par.oracle_step(oracle.Oracle(), c, accept=acc_r)
    par.assert_states_match(c, ref)
