"""The oracle's steps composed on the small one-request workload (N = 512, G = 4): tiers,
allocation, page images and attention read back from the images."""
import numpy as np

from oracle import attention as oatt, layout, place, pool as opool, score as osc
from mixed_precision_paged_score_amd import workloads


def test_workload1_end_to_end():
    w = workloads.workload(1)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k).numpy()
    k, v = k.numpy(), v.numpy()
    tier, count, _ = osc.score_tokens(acc, w.cu_seqlens(), w.num_kv_heads, w.alpha_h,
                                      w.alpha_l, w.window)
    # random queries under a causal softmax put almost every token above 1/N
    assert (tier == osc.HIGH).mean() > 0.9
    pl = opool.Pool(1, 1, w.num_kv_heads, w.row_capacity, w.num_pages)
    pl.compact(0, count)
    pl.check_invariants()
    q = workloads.make_queries(w).numpy()
    G = w.group
    for h in range(w.num_kv_heads):
        imgs = place.head_pages(k[:, h], v[:, h], tier[:, h])
        qH, qL = opool.pages_needed(*count[0, h])
        assert len(imgs[place.HIGH]) == qH and len(imgs[place.LOW]) == qL
        kh, vh = place.dequantize_pages(imgs[place.HIGH], place.HIGH, count[0, h, 0])
        kl, vl = place.dequantize_pages(imgs[place.LOW], place.LOW, count[0, h, 1])
        kd, vd = place.head_dequantized(k[:, h], v[:, h], tier[:, h])
        assert np.array_equal(np.concatenate([kh, kl]), kd)
        assert np.array_equal(np.concatenate([vh, vl]), vd)
        # positions stored in the pages are the tokens' positions, ascending per tier
        for t, imgl in ((place.HIGH, imgs[place.HIGH]), (place.LOW, imgs[place.LOW])):
            n = count[0, h, 0 if t == place.HIGH else 1]
            got = np.concatenate([layout.read_page(img, t, min(layout.SLOTS[t], n - i * layout.SLOTS[t]))[6]
                                  for i, img in enumerate(imgl)]) if imgl else np.zeros(0)
            assert np.array_equal(got, np.nonzero(tier[:, h] == t)[0])
        o = oatt.decode_group(q[0, h * G:(h + 1) * G], kd, vd, 128 ** -0.5)
        # quantization error stays small against full-precision attention
        o_ref = oatt.decode_group(q[0, h * G:(h + 1) * G], k[:, h].astype(np.float32),
                                  v[:, h].astype(np.float32), 128 ** -0.5)
        assert np.abs(o - o_ref).max() < 0.1
