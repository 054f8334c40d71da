"""The decode entry point that allocates nothing (tq_decode_attention_static,
scratch in the library's static per-GPU array) against tq_decode_attention
(scratch in the arena's workspace), through the C ABI: two twin caches fed
the same tokens, one driven through each entry point, two calls in a row
with the second smaller (the first call's records stay in the static array),
promotion after each; outputs within the 2e-3 bar (the same kernels run, so
they are expected to agree exactly) and the paging state equal."""

import numpy as np
import pytest

from compressed_kv_decode_amd import workloads as wl

from gpu_helpers import OUT_ATOL, dev, make_cache

pytestmark = pytest.mark.gpu


def test_static_workspace_entry_point_matches_arena_entry_point():
    import torch
    w = wl.make("llama8b").with_(n_seq=4, n_layers=2, prefill=(5000, 3100, 4500, 1289), formats=(wl.F3, wl.F4),
                                 steps=2, tau=0.15, sticky=1, heavy_hitters=2)
    caches = [make_cache(w), make_cache(w)]  # 0: arena workspace, 1: static workspace
    seqs = list(range(w.n_seq))
    for layer in range(w.n_layers):
        ks, vs = zip(*[wl.prefill_kv(w, layer, sq) for sq in seqs])
        for c in caches:
            c.append(layer, seqs, list(w.prefill), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    # call 1: layer 0, every sequence; call 2: layer 1, two sequences
    for layer, ids in ((0, seqs), (1, [1, 3])):
        sk, sv = zip(*[wl.step_kv(w, layer, sq, 0) for sq in ids])
        q = dev(np.stack([wl.query(w, layer, sq, 1) for sq in ids]))  # a heavy-hitter step
        outs, lgs = [], []
        for i, c in enumerate(caches):
            c.append(layer, ids, [1] * len(ids), dev(np.concatenate(sk)), dev(np.concatenate(sv)))
            lg = torch.full((len(ids), w.n_q_heads, c.logits_stride), float("nan"), device="cuda")
            outs.append(c.attend(layer, ids, q, static_workspace=bool(i)).cpu().numpy())
            c.attend(layer, ids, q, logits=lg, static_workspace=bool(i))
            lgs.append(lg.cpu().numpy())
            c.promote(layer, ids)
        torch.cuda.synchronize()
        err = float(np.abs(outs[1] - outs[0]).max())
        print(f"layer {layer}, {len(ids)} sequences: static vs arena output max-abs {err:.3e}", flush=True)
        assert err <= OUT_ATOL
        assert np.array_equal(np.isfinite(lgs[0]), np.isfinite(lgs[1]))
        fin = np.isfinite(lgs[0])
        assert np.abs(lgs[1][fin] - lgs[0][fin]).max() <= 1e-3 * max(1.0, np.abs(lgs[0][fin]).max())
        promoted = 0
        for sq in ids:
            a, b = (c.export_hot(sq, layer) for c in caches)
            assert a[0] == b[0], f"seq {sq} layer {layer}: hot FIFO tags differ"
            assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
            n = caches[0].stats(sq, layer)["cold_len"]
            pa, pb = (c.export_paging(sq, layer, n) for c in caches)
            assert np.array_equal(pa[0], pb[0]) and np.array_equal(pa[1], pb[1])
            promoted += sum(t >= 0 for t in a[0])
        assert promoted >= 1, "the heavy-hitter step promotes through both entry points"
