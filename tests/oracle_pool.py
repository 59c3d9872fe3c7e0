"""Oracle row chunks in worker processes.  TEST INFRASTRUCTURE ONLY.

The oracle is plain numpy with a Python loop over 128-key tiles and 32-key
blocks, so threads serialize on the interpreter lock.  The full-size parity
checks therefore run it in separate processes, started with "spawn": they
import numpy, the oracle and the comparison helpers, never torch, and never
touch the GPU.  Each (sequence, KV head) reaches them as a file of its bf16
K and V rows (as float32) under /dev/shm, which each worker quantizes once
and keeps; each task carries one chunk of query rows and the kernel's
outputs and probability dump for those rows.
"""

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from helpers import (assert_close_outputs, check_code_choices, gpu_codes, oracle_prepare_kv, oracle_prepare_q,
                     p_mismatch, tie_flip_bound)
from oracle import attention as OA

WORKERS = max(1, min(16, os.cpu_count() or 1))
_pool = None
_kv_cache = {}
_limits = None


def _init_worker():
    global _limits
    from threadpoolctl import threadpool_limits
    _limits = threadpool_limits(limits=1)      # one BLAS thread per worker process


def pool():
    """The shared worker pool (started on first use)."""
    global _pool
    if _pool is None:
        _pool = ProcessPoolExecutor(max_workers=WORKERS, mp_context=mp.get_context("spawn"),
                                    initializer=_init_worker)
    return _pool


def shutdown():
    global _pool
    if _pool is not None:
        _pool.shutdown()
        _pool = None


def _kv(path, params):
    if path not in _kv_cache:
        if len(_kv_cache) >= 4:
            _kv_cache.clear()
        with np.load(path) as z:
            k, v = z["k"], z["v"]
        _kv_cache[path] = oracle_prepare_kv(k, v, **params)
    return _kv_cache[path]


def fwd_chunk(t):
    """One chunk of query rows of one (sequence, head): the oracle's forward
    with its unrounded values, the oracle-only near-tie bound, and -- with a
    dump -- the code checks and the comparison on the kernel's codes.  Returns
    the oracle's O / LSE and bounds (the caller adds them to its PureCompare)
    with the counts."""
    k_raw, gk, v_hat = _kv(t["kv_path"], t["kv_params"])
    q_raw, gq, sig = oracle_prepare_q(t["q"], **t["q_params"])
    L, rc, pf, enc, causal = t["L"], t["rows"], t["p_format"], t["encoder"], t["causal"]
    O, Lr, oc, oe, pre, xmax, tiles = OA.attn_lowp_head(q_raw, k_raw, gq, gk, v_hat, sig, pf, causal, q_index=rc,
                                                         encoder=enc, return_pre=True, return_tiles=True)
    live = np.arange(L)[None, :] <= rc[:, None] if causal else np.ones((len(rc), L), bool)
    ob, lb, _ = tie_flip_bound(pre, oc, oe, xmax, tiles, O, v_hat, pf, enc, live)
    out = dict(O=O, L=Lr, ob=ob, lb=lb, n_e=0, n_c=0, mis=0, tot=0, tight=None)
    if t["dc"] is not None:
        gc, ge = gpu_codes(t["dc"], t["ds"], pf, L)
        n_e, n_c = check_code_choices(gc, ge, oc, oe, pre, xmax, pf, enc, live)
        mis, tot = p_mismatch(t["dc"], t["ds"], oc, oe, pf, L, live)
        out.update(n_e=n_e, n_c=n_c, mis=mis, tot=tot)
        if n_e or n_c:
            O2, L2 = OA.attn_lowp_head(q_raw, k_raw, gq, gk, v_hat, sig, pf, causal, q_index=rc, encoder=enc,
                                       p_given=(gc, ge))
            out["tight"] = assert_close_outputs(t["og"], t["lg"], O2, L2, f"{t['what']} on the kernel's codes")
    return out
