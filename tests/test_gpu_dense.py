"""GPU parity of the dense fp32 GDN / KDA decode step against the fp64 oracle.

Tolerance: norm-wise relative error 1e-5 for every (head, step) output and for
the final state, as fixed for fp32 state and outputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import DEV, TOL_F32, dev_inputs, rel_err, rsu, run_dense, say

pytestmark = pytest.mark.gpu


def test_gdn_b4_h8_f32_all_heads_64_steps():
    w = wl.WORKLOADS[1]
    say(f"[dense] {w.name}: B={w.B} H={w.H} steps={w.steps} all heads")
    ey, eS = run_dense(w)
    say(f"[dense] {w.name}: max rel err y={ey:.3e} S={eS:.3e}")
    assert ey < TOL_F32 and eS < TOL_F32


@pytest.mark.parametrize("variant,qkv,B,H", [("gdn", "bf16", 3, 7), ("kda", "f32", 5, 3), ("gdn", "bf16", 10, 10),
                                             ("kda", "bf16", 1, 1), ("gdn", "f32", 2, 1)])
def test_ragged_small_batches(variant, qkv, B, H):
    base = wl.WORKLOADS[3] if variant == "kda" else wl.WORKLOADS[2]
    w = wl.custom(base, B=B, H=H, qkv=qkv, steps=12)
    say(f"[dense] ragged {variant} {qkv} B={B} H={H}")
    ey, eS = run_dense(w)
    assert ey < TOL_F32 and eS < TOL_F32


def test_gdn_b256_h48_bf16_full_size_sampled():
    """Serving-scale GDN workload in the launch configuration the benchmark times."""
    w = wl.WORKLOADS[2]
    say(f"[dense] {w.name}: full size, 96 sampled heads, {w.steps} steps")
    ey, eS = run_dense(w, sample=96)
    say(f"[dense] {w.name}: max rel err y={ey:.3e} S={eS:.3e}")
    assert ey < TOL_F32 and eS < TOL_F32


def test_kda_b128_h32_bf16_full_size_sampled():
    w = wl.WORKLOADS[3]
    say(f"[dense] {w.name}: full size, 96 sampled heads, {w.steps} steps")
    ey, eS = run_dense(w, sample=96)
    say(f"[dense] {w.name}: max rel err y={ey:.3e} S={eS:.3e}")
    assert ey < TOL_F32 and eS < TOL_F32


@pytest.mark.parametrize("kda", [False, True])
def test_identity_step_leaves_state_bit_exact(kda):
    m = rsu()
    B, H = 2, 3
    g = torch.Generator().manual_seed(5)
    S0 = torch.randn(B, H, 128, 128, generator=g).to(DEV)
    S = S0.clone()
    q = torch.nn.functional.normalize(torch.randn(B, H, 128, generator=g), dim=-1).to(DEV)
    k = torch.nn.functional.normalize(torch.randn(B, H, 128, generator=g), dim=-1).to(DEV)
    v = torch.randn(B, H, 128, generator=g).to(DEV)
    gate = torch.ones((B, H, 128) if kda else (B, H), device=DEV)
    beta = torch.zeros(B, H, device=DEV)
    y = torch.empty(B, H, 128, device=DEV)
    (m.kda_decode_step if kda else m.gdn_decode_step)(S, q, k, v, gate, beta, y)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    ref = np.einsum("bhij,bhi->bhj", S0.double().cpu().numpy(), q.double().cpu().numpy())
    assert rel_err(y.cpu().numpy().reshape(-1, 128), ref.reshape(-1, 128)) < TOL_F32


def test_unit_key_writes_value():
    """alpha = beta = 1, unit k, q = k: the post-update readout returns v."""
    m = rsu()
    B, H = 4, 5
    g = torch.Generator().manual_seed(6)
    S = (torch.randn(B, H, 128, 128, generator=g) * 0.3).to(DEV)
    k = torch.nn.functional.normalize(torch.randn(B, H, 128, generator=g, dtype=torch.float64),
                                      dim=-1).float().to(DEV)
    v = torch.randn(B, H, 128, generator=g).to(DEV)
    y = torch.empty(B, H, 128, device=DEV)
    m.gdn_decode_step(S, k, k, v, torch.ones(B, H, device=DEV), torch.ones(B, H, device=DEV), y)
    assert rel_err(y.cpu().numpy().reshape(-1, 128), v.cpu().numpy().reshape(-1, 128)) < 1e-5


def test_empty_batch_and_errors():
    m = rsu()
    e = torch.empty(0, 48, 128, device=DEV)
    m.gdn_decode_step(torch.empty(0, 48, 128, 128, device=DEV), e, e, e,
                      torch.empty(0, 48, device=DEV), torch.empty(0, 48, device=DEV), e.clone())
    with pytest.raises(ValueError):
        m.gdn_decode_step(torch.empty(1, 1, 64, 64, device=DEV), *([torch.empty(1, 1, 128, device=DEV)] * 3),
                          torch.empty(1, 1, device=DEV), torch.empty(1, 1, device=DEV),
                          torch.empty(1, 1, 128, device=DEV))


def test_bitwise_deterministic():
    w = wl.custom(wl.WORKLOADS[2], B=8, H=8, steps=3)
    m = rsu()
    outs = []
    for _ in range(2):
        S = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
        y = torch.empty(w.B, w.H, 128, device=DEV)
        for t in range(w.steps):
            _, d = dev_inputs(w, t)
            m.gdn_decode_step(S, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        outs.append((S.clone(), y.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_copy_probe_copies():
    m = rsu()
    n = 128 * 128 * 3 + 100
    src = torch.randn(n, device=DEV)
    dst = torch.zeros(n, device=DEV)
    m.copy_f32(src, dst)
    assert torch.equal(src, dst)


def test_stream_probes_read_and_write_every_tile():
    """The HBM ceiling probes touch every element: the read probe's column sums equal
    torch's, the write probe fills every element (over a full block of the XCD-grouped
    tile order plus a ragged tail)."""
    m = rsu()
    tiles = 32 + 5
    src = torch.randn(tiles, 128, 128, device=DEV)
    sums = torch.zeros(tiles, 128, device=DEV)
    m.read_f32(src, sums)
    torch.testing.assert_close(sums, src.sum(dim=1), rtol=1e-5, atol=1e-4)
    dst = torch.zeros(tiles, 128, 128, device=DEV)
    m.fill_f32(dst, 0.75)
    assert bool((dst == 0.75).all())

