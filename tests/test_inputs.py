"""The seeded input generator: packing bounds, the neuron-major relayout, determinism."""
import numpy as np
import torch

import moe_inputs as mi
from tests import bruteforce as bf


def test_q8_0_pack_error_is_at_most_half_a_step():
    g = torch.Generator().manual_seed(1)
    w = torch.randn((7, 96), generator=g) * 0.02
    q, d = mi.pack_q8_0(w)
    deq = q.double() * torch.repeat_interleave(d.double(), 32, dim=-1)
    step = torch.repeat_interleave(d.double(), 32, dim=-1)
    assert torch.all((deq - w.double()).abs() <= step / 2 + 1e-12)
    assert q.abs().max() <= 127
    q0, d0 = mi.pack_q8_0(torch.zeros((2, 64)))
    assert torch.all(q0 == 0) and torch.all(d0 == 0)


def test_i8_row_pack_error_is_at_most_half_a_step():
    g = torch.Generator().manual_seed(2)
    w = torch.randn((9, 80), generator=g)
    q, s = mi.pack_i8_row(w)
    deq = q.double() * s.double()[:, None]
    assert torch.all((deq - w.double()).abs() <= s.double()[:, None] / 2 * (1 + 1e-6))


def test_e2m1_pack_picks_the_nearest_value_and_packs_low_nibble_first():
    tab = bf.e2m1_table()
    g = torch.Generator().manual_seed(3)
    w = torch.randn((5, 64), generator=g)
    packed, s16, codes = mi.pack_e2m1_g16(w)
    assert torch.equal(packed, codes[:, 0::2] | (codes[:, 1::2] << 4))
    s = torch.repeat_interleave(s16.double(), 16, dim=-1).numpy()
    r = w.double().numpy() / s
    got = tab[codes.numpy()]
    best = np.abs(r[..., None] - tab[None, None, :]).min(-1)
    assert np.allclose(np.abs(r - got), best, atol=1e-12)
    # exact midpoints go to the even code
    mid = torch.tensor([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 6, 0, 0, 0, 0, 0, 0, 0]]) * 1.0
    _, s_mid, c_mid = mi.pack_e2m1_g16(mid)
    assert s_mid.item() == 1.0
    assert c_mid[0, :8].tolist() == [0, 2, 2, 4, 4, 6, 6, 14]


def test_neuron_major_relayout_is_a_pure_permutation():
    w = mi.workload("nemotron_latent", E=2, d_model=64, d_ff=48, k=1, T=1)
    g = torch.Generator().manual_seed(4)
    wd = torch.randn((2, 64, 48), generator=g) * 0.02
    _, s16, codes = mi.pack_e2m1_g16(wd)
    V, S = mi.neuron_major_down(codes, s16)
    assert V.numel() * 2 == codes.numel() and S.numel() == s16.numel()   # same size
    for e in range(2):
        for f in range(48):
            for o in range(64):
                b = int(V[e, f, o // 2])
                c = (b >> 4) if o % 2 else (b & 15)
                assert c == int(codes[e, o, f])
            for o in range(64):
                assert S[e, f // 16, o] == s16[e, o, f // 16]


def test_generator_is_deterministic_and_seeds_differ_per_instance():
    w = mi.workload("tiny")
    a = mi.make_layer(w, 0)
    b = mi.make_layer(w, 0)
    c = mi.make_layer(w, 1)
    for key in ("gate_up", "gate_up_scales", "down", "down_scales"):
        assert torch.equal(a["experts"][key], b["experts"][key])
        assert not torch.equal(a["experts"][key], c["experts"][key])
    assert torch.equal(mi.make_x(w, 0), mi.make_x(w, 0))
    assert mi.base_seed(w, 0) == 0


def test_workload_shapes():
    assert mi.expert_bytes(mi.workload("gemma_decode")) == 6_319_104
    assert mi.expert_bytes(mi.workload("gemma_decode", fmt=mi.FMT_I8_ROW)) == 5_964_288
    assert mi.expert_bytes(mi.workload("m3_decode")) == 60_162_048
    assert mi.expert_bytes(mi.workload("nemotron_latent")) == 3_440_640
    assert mi.expert_bytes(mi.workload("tiny")) == 417_792


def test_latent_bias_column_construction():
    w = mi.workload("nemotron_latent", E=2, k=1, T=2)
    x = mi.make_x(w, 0)
    assert torch.all(x[:, -1].float() == 1.0)
    lay = mi.make_layer(w, 0)
    ex = lay["experts"]
    code_last = (ex["gate_up"][:, :, -1] >> 4)          # element d-1 is the high nibble
    s_last = ex["gate_up_scales"][:, :, -1].float()
    assert torch.all(code_last == 15)                     # -6: the block's largest magnitude
    ref = 1.44 * 0.02 * (1023 ** 0.5)
    assert torch.allclose(6 * s_last, torch.full_like(s_last, ref), rtol=1e-3)
