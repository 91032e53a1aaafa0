"""The seeded input generators: deterministic, right shapes and distributions."""
import numpy as np
import torch

import synth


def test_workload_table_shapes_and_flops():
    w5 = synth.WORKLOADS[5]
    assert [l.name for l in w5.linears] == ["qkv", "o", "gate", "up", "down"]
    assert abs(w5.flops() / 1e9 - 14018.77) < 0.01      # 2*M*N*K summed
    assert abs(synth.WORKLOADS[2].flops() / 1e9 - 79.73) < 0.01
    assert abs(synth.WORKLOADS[3].flops() / 1e9 - 1108.10) < 0.01
    assert abs(synth.WORKLOADS[4].flops() / 1e9 - 3478.92) < 0.01
    for w in synth.WORKLOADS.values():
        for l in w.linears:
            assert w.tensor(l.x).shape == (l.M, l.K)
            assert w.tensor(l.w).shape == (l.N, l.K)
            if l.dy:
                assert w.tensor(l.dy).shape == (l.M, l.N)


def test_generators_are_deterministic_and_seeded_per_tensor():
    w = synth.WORKLOADS[1]
    a = synth.workload_tensor(w, "X")
    b = synth.workload_tensor(w, "X")
    assert a.dtype == torch.bfloat16 and a.shape == (128, 256)
    assert synth.sha256(a) == synth.sha256(b)
    assert synth.sha256(a) != synth.sha256(synth.workload_tensor(w, "W"))
    assert w.seed("X") == 1000 and w.seed("W") == 1001


def test_distributions():
    x = synth.draw_f32(5, (1000, 1000), "normal", 0.02)
    assert abs(x.std() - 0.02) < 2e-4 and abs(x.mean()) < 1e-4
    t = synth.draw_f32(6, (1000, 1000), "t3_outliers", 1.0)
    big = int((np.abs(t) > 50).sum())              # nearly all of these are the x100 outliers
    assert 500 < big < 1000                        # 1000 outliers, most with |t3| > 0.5
    assert np.median(np.abs(t)) < 1.0
    bf = synth.to_bf16(np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32))
    assert bf.float().tolist() == [1.0, 1.0 + 2 ** -6]   # nearest-even to 7 fraction bits


def test_chained_mlp_workload():
    m = synth.CHAINED_MLPS[6]
    assert (m.tokens, m.d, m.f) == (4096, 4096, 11008)
    assert m.shape("W1") == (2 * 11008, 4096) and m.shape("W2") == (4096, 11008)
    assert m.flops() == 18 * 4096 * 11008 * 4096          # 3 forward-shaped products x 3 passes
    assert [m.seed(n) for n in m.ORDER] == [6000, 6001, 6002, 6003]
    small = synth.ChainedMLP(77, "t", 8, 16, 12)
    x = synth.chained_mlp_tensor(small, "X")
    w1 = synth.chained_mlp_tensor(small, "W1")
    g = synth.chained_mlp_tensor(small, "G")
    assert x.dtype == torch.bfloat16 and x.shape == (8, 16)
    assert w1.dtype == torch.float32 and w1.shape == (24, 16)
    assert g.dtype == torch.float32 and abs(float(g.std()) - 1e-6) < 5e-7
    assert synth.sha256(x) == synth.sha256(synth.chained_mlp_tensor(small, "X"))
