"""The seeded input generators (no method arithmetic): the generation-round accumulators keep
their meaning, the sum of the weight each token received from strictly later queries."""
import dataclasses

import numpy as np
import torch

from mixed_precision_paged_score_amd import workloads


def test_round_accumulators_add_the_rounds_weights():
    w0 = workloads.Workload("acc-round", 1, 3, 8, 2, [50, 1, 0], 1.0, 0.2, 4, 512, "zipf",
                            seed=5)
    acc0 = workloads.make_acc(w0)
    grow = 7
    w1 = dataclasses.replace(w0, seqlens=[n + grow for n in w0.seqlens], seed=99)
    acc1 = workloads.make_acc_zipf_round(w1, acc0, w0.seqlens, "cpu", 1)
    cu0, cu1 = w0.cu_seqlens(), w1.cu_seqlens()
    s = 1.1
    for b in range(w0.batch):
        n0, n = w0.seqlens[b], w1.seqlens[b]
        inc = acc1[cu1[b]:cu1[b + 1]].double().numpy()
        inc[:n0] -= acc0[cu0[b]:cu0[b + 1]].double().numpy()
        later = np.where(np.arange(n) < n0, n - n0, n - 1 - np.arange(n)).astype(np.float64)
        assert later[-1] == 0 and np.all(inc[-1] == 0)        # nothing follows the last token
        # the per-position mean weights of every query head are a permutation of the Zipf law
        m = inc[later > 0] / later[later > 0, None]
        zipf = np.arange(1, n + 1, dtype=np.float64) ** -s
        zipf /= zipf.sum()
        for hq in range(w1.num_q_heads):
            got = np.sort(m[:, hq])
            # each one of the law's values (the last position's value is not observed), up to
            # the float32 rounding of the stored sums
            near = np.abs(got[:, None] - zipf[None, :]).min(axis=1)
            assert np.all(near <= 1e-5 * got + 1e-9), near.max()
            assert len(np.unique(np.round(got / got.max(), 5))) == len(got)   # no value twice
            assert got.sum() <= 1.0 + 1e-6


def test_round_accumulators_are_seeded():
    w0 = workloads.Workload("acc-seed", 1, 2, 4, 1, [30, 9], 1.0, 0.2, 4, 512, "zipf", seed=8)
    acc0 = workloads.make_acc(w0)
    w1 = dataclasses.replace(w0, seqlens=[40, 19], seed=77)
    a = workloads.make_acc_zipf_round(w1, acc0, w0.seqlens, "cpu", 3)
    b = workloads.make_acc_zipf_round(w1, acc0, w0.seqlens, "cpu", 3)
    c = workloads.make_acc_zipf_round(w1, acc0, w0.seqlens, "cpu", 4)
    assert torch.equal(a, b) and not torch.equal(a, c)
