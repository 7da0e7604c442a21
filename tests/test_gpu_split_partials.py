"""Split-KV partial results of the HIP path against the oracle.

Every split of a split stream carries, per query row and head, the base-2
log-sum-exp of the scores over exactly its tokens and its normalised output
over them ([p5] "How Paged KV Cache Attention Achieves Stable Inference in
Ling-Bot-Map" §Kernel Dispatch and Sequence Lengths: the splits combine to
the exact softmax over the valid tokens).  The split's tokens are read off
the plan image (its unit range) and gathered from the oracle's own pool; the
log-sum-exp is compared with the oracle's lse_base2_fp64 over them, the
output with attention_fp64 over them."""
import dataclasses

import numpy as np
import pytest

import kvc_synth as syn
from oracle import kvc_oracle as ko
from tests.stream_harness import Harness, check_close

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

HEADER, REC = 8, 20
F_UNIT0, F_NUNITS, F_NSPLIT, F_QTILE0, F_NQ = 7, 8, 9, 15, 1
# A wrong split boundary (one 64-slot unit more or less) moves the
# log-sum-exp by log2(1 +- 64 / L_split), above 0.05 at every checked split;
# the kernel's own error (probabilities rounded to the element type before
# their sum) stays below 0.01.
LSE_BOUND = 2.0 ** -6


def split_tokens(img, rec0, split, pool, page_size):
    n_units, n_split, unit0 = (int(img[rec0 + f]) for f in (F_NUNITS, F_NSPLIT, F_UNIT0))
    u0, u1 = split * n_units // n_split, (split + 1) * n_units // n_split
    ks, vs = [], []
    for u in range(u0, u1):
        slot, valid = int(img[unit0 + 4 * u]) & 0xFFFFFFFF, int(img[unit0 + 4 * u + 1])
        page, off = divmod(slot, 2 * page_size)
        ks.append(pool[page, 0, off:off + valid])
        vs.append(pool[page, 1, off:off + valid])
    return np.concatenate(ks), np.concatenate(vs)


def partial_output(o, split, head, tile0, n_q, D):
    """[n_q, D] raw 16-bit values of one split's normalised output."""
    out = np.zeros((n_q, D), np.uint16)
    for r in range(n_q):
        t, r32 = divmod(r, 32)
        for d in range(D):
            out[r, d] = o[split, head, tile0 + t, d // 32, (d % 32) // 8, 32 * ((d % 8) // 4) + r32, d % 4]
    return out


def check_splits(h, res, wl, max_splits_checked=None, label=""):
    lse, o = h.gpu.get_split_partials()
    img = h.gpu.get_plan_image().astype(np.int64)
    q = res["q_bits"][0]
    pool = h.ora.pools[0].data
    rec0 = HEADER
    n_split, tile0, n_q = (int(img[rec0 + f]) for f in (F_NSPLIT, F_QTILE0, F_NQ))
    assert n_split > 1, "the checked step must split the stream"
    splits = range(n_split) if max_splits_checked is None else \
        sorted(set(np.linspace(0, n_split - 1, max_splits_checked).astype(int)))
    worst = 0.0
    for s in splits:
        k, v = split_tokens(img, rec0, s, pool, wl.page_size)
        ref_lse = ko.lse_base2_fp64(q, k, wl.dtype)                       # [T, H]
        ref_o = ko.attention_fp64(q, k, v, wl.dtype)                      # [T, H, D]
        got_lse = lse[s, :, tile0:tile0 + (n_q + 31) // 32, :].reshape(wl.num_heads, -1)[:, :n_q].T
        err = np.abs(got_lse.astype(np.float64) - ref_lse)
        worst = max(worst, float(err.max()))
        assert err.max() <= LSE_BOUND, (label, s, float(err.max()))
        got_o = np.stack([partial_output(o, s, hd, tile0, n_q, wl.head_dim) for hd in range(wl.num_heads)], axis=1)
        check_close(got_o, ref_o, dtype=wl.dtype)
    print(f"{label}: {n_split} splits, {len(splits)} checked, max |lse error| {worst:.2e}", flush=True)


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_split_partials_tiny_every_split():
    """Head size 32, 2 heads, 16-slot pages: every split at the last step."""
    _need_gpu()
    wl = syn.WORKLOADS["tiny"]
    h = Harness(wl)
    F = max(wl.frames)
    for t in range(F):
        res = h.step(run=t == F - 1)
    check_splits(h, res, wl, label="tiny")


def test_split_partials_base_shape():
    """Head size 64 at the measured shape (262 queries: 8 tiles and a 6-row
    tail), 4 heads, 80 frames; a spread of the splits."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(80,))
    h = Harness(wl)
    F = max(wl.frames)
    for t in range(F):
        res = h.step(run=t == F - 1)
    check_splits(h, res, wl, max_splits_checked=6, label="base H=4")
