"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI
binding and compare with the float64 oracle under the accuracy rule."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from workloads import make_inputs

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def to_dev(*ts):
    return [None if t is None else t.cuda() for t in ts]


def run_gpu(mha, q, k, v, kl, causal, variant="auto"):
    qd, kd, vd, kld = to_dev(q, k, v, kl)
    out, lse = mha.forward(qd, kd, vd, causal=causal, key_len=kld, variant=variant)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check_full(out, lse, q, k, v, kl, causal, label=""):
    """Every element of out and lse against the oracle; returns budget fractions."""
    ro, rl = oracle.attention(q, k, v, causal=causal, key_len=kl, threads=THREADS)
    ok_o = oracle.gate(out, ro)
    ok_l = oracle.gate(lse, rl)
    fo, fl = oracle.budget_fraction(out, ro), oracle.budget_fraction(lse, rl)
    if not (ok_o.all() and ok_l.all()):
        bad = np.argwhere(~ok_o)[:5].tolist()
        badl = np.argwhere(~ok_l)[:5].tolist()
        raise AssertionError(
            f"{label}: {int((~ok_o).sum())} out / {int((~ok_l).sum())} lse elements fail the rule; "
            f"out budget {fo:.3f} lse budget {fl:.3f}; first bad out {bad} lse {badl}")
    return fo, fl


def check_rows(out, lse, q, k, v, kl, causal, rows, label=""):
    """Sampled (b, h, i) rows of out / lse against exact oracle rows."""
    ro, rl = oracle.attention_rows(q, k, v, rows, causal=causal, key_len=kl)
    idx = (torch.as_tensor(rows[:, 0]), torch.as_tensor(rows[:, 1]), torch.as_tensor(rows[:, 2]))
    uo = out[idx].cpu() if out.is_cuda else out[idx]
    ul = lse[idx].cpu() if lse.is_cuda else lse[idx]
    ok_o, ok_l = oracle.gate(uo, ro), oracle.gate(ul, rl)
    fo, fl = oracle.budget_fraction(uo, ro), oracle.budget_fraction(ul, rl)
    if not (ok_o.all() and ok_l.all()):
        bad = rows[np.argwhere(~ok_o.all(axis=-1))[:5, 0]].tolist()
        raise AssertionError(f"{label}: sampled rows fail the rule (out budget {fo:.3f}, "
                             f"lse budget {fl:.3f}); first bad rows {bad}")
    return fo, fl


def workload_case(mha, w, seed, variant="auto", label=None):
    q, k, v, kl = make_inputs(w, seed)
    out, lse = run_gpu(mha, q, k, v, kl, w.causal, variant)
    return check_full(out, lse, q, k, v, kl, w.causal, label or f"{w.name} seed {seed} {variant}")


def check_full_chunked(out, lse, q, k, v, kl, causal, label="", chunk=625):
    """check_full over batch chunks run on THREADS host threads: the same
    oracle and the same rule on every element, in pieces small enough for a
    full-size launch (numpy releases the interpreter lock in its array work)."""
    B = q.shape[0]

    def one(b0):
        b1 = min(B, b0 + chunk)
        klc = None if kl is None else kl[b0:b1]
        ro, rl = oracle.attention(q[b0:b1], k[b0:b1], v[b0:b1], causal=causal, key_len=klc, threads=1)
        uo, ul = out[b0:b1], lse[b0:b1]
        ok_o, ok_l = oracle.gate(uo, ro), oracle.gate(ul, rl)
        nbad = int((~ok_o).sum()) + int((~ok_l).sum())
        first = None
        if nbad:
            bad = np.argwhere(~ok_o)
            first = (bad[:3] + np.array([b0, 0, 0, 0])).tolist() if len(bad) else None
        return nbad, first, oracle.budget_fraction(uo, ro), oracle.budget_fraction(ul, rl)

    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(one, range(0, B, chunk)))
    nbad = sum(r[0] for r in res)
    fo, fl = max(r[2] for r in res), max(r[3] for r in res)
    if nbad:
        first = [r[1] for r in res if r[1]][:1]
        raise AssertionError(f"{label}: {nbad} elements fail the rule; out budget {fo:.3f} "
                             f"lse budget {fl:.3f}; first bad out {first}")
    return fo, fl
