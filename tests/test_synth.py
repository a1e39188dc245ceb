"""The seeded workload generator: determinism and the shapes of the configs."""

import numpy as np

import synth


def test_deterministic():
    a = synth.make(synth.SMALL[3])
    b = synth.make(synth.SMALL[3])
    assert (a.context_lens == b.context_lens).all() and (a.free_order == b.free_order).all()
    assert a.q.tobytes() == b.q.tobytes()
    assert a.values(("seq", 2), 0, 5)[0].tobytes() == b.values(("seq", 2), 0, 5)[0].tobytes()


def test_full_config_shapes():
    c1 = synth.make(1)
    assert list(c1.context_lens) == [1, 17, 33, 100] and c1.num_blocks == 64
    assert sorted(c1.free_order) == list(range(64))
    c3 = synth.make(3)
    assert c3.context_lens.min() >= 512 and c3.context_lens.max() <= 8192 and len(c3.context_lens) == 64
    assert c3.num_blocks == 2 * int(((c3.context_lens + 15) // 16).sum())
    c4 = synth.make(4)
    assert (c4.context_lens >= 1030 + 16).all() and (c4.context_lens <= 1030 + 512).all()
    c5 = synth.make(5)
    L = c5.context_lens
    assert (L[:8] >= 32768).all() and (L[:8] <= 131072).all()
    assert (L[8:] >= 64).all() and (L[8:] <= 512).all() and len(L) == 256


def test_ops_cover_every_token_once():
    for k in (1, 2, 3, 4, 5):
        wl = synth.make(synth.SMALL[k])
        c = wl.cfg
        per_seq = np.zeros(c.S, dtype=np.int64)
        shared = 0
        for op in wl.prefill + wl.decode:
            if op[0] == "append":
                if op[3][0] == "prefix":
                    shared += op[2]
                else:
                    per_seq[op[1]] += op[2]
        assert ((per_seq + (c.prefix if c.prefix else 0)) == wl.context_lens).all()
        assert len(wl.decode) == c.S and all(op[2] == 1 for op in wl.decode)
