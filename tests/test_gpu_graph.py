"""The C-ABI calls captured in a HIP graph (torch.cuda.graph) and replayed give the same
results, bit for bit, as the same calls launched one by one.

Each case keeps two copies of the buffers. The graph is captured once on copy B (capturing
runs nothing); then, three times over, the same block of steps runs eagerly on copy A and
the graph is replayed on copy B, with a synchronization and a comparison of every buffer
and output after each round. The calls launch only the library's own kernels (no memset
nodes), so every replay must match.
"""
import pytest
import torch

import workloads as wl
from parity import DEV, dev_inputs, log_step, new_lq_buffers, new_log_buffers, new_window_buffers, rsu, window_step

pytestmark = pytest.mark.gpu


def _twin(bufs):
    return {k: v.clone() for k, v in bufs.items()}


def _check_rounds(run_block, bufs_a, bufs_b, y_a, y_b, rounds=3):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_block(bufs_b, y_b)
    torch.cuda.synchronize()
    for r in range(rounds):
        run_block(bufs_a, y_a)   # eager
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in bufs_a:
            assert torch.equal(bufs_a[k], bufs_b[k]), f"round {r}: {k} differs"
        assert torch.equal(y_a, y_b), f"round {r}: y differs"


def test_graph_dense_gdn():
    m = rsu()
    w = wl.custom(wl.WORKLOADS[2], B=3, H=5)
    S = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    ins = [dev_inputs(w, t)[1] for t in range(4)]

    def block(b, y):
        for d in ins:
            m.gdn_decode_step(b["S"], d["q"], d["k"], d["v"], d["gate"], d["beta"], y)

    a, b = {"S": S.clone()}, {"S": S.clone()}
    _check_rounds(block, a, b, torch.zeros(w.B, w.H, 128, device=DEV), torch.zeros(w.B, w.H, 128, device=DEV))


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_graph_int8_window(variant):
    """Two whole windows of W = 4 per block: in-window steps and boundaries."""
    m = rsu()
    base = wl.WORKLOADS[4] if variant == "gdn" else wl.custom(wl.WORKLOADS[4], variant="kda", gate_lo=0.8, gate_hi=1.0)
    w = wl.custom(base, B=2, H=7, W=4)
    bufs = new_window_buffers(w)
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    m.q8_quantize(S0, bufs["Z"], bufs["A"])
    ins = [dev_inputs(w, t)[1] for t in range(2 * w.W)]

    def block(b, y):
        for t, d in enumerate(ins):
            window_step(w, t % w.W, b, d, y)

    _check_rounds(block, _twin(bufs), _twin(bufs), torch.zeros(w.B, w.H, 128, device=DEV),
                  torch.zeros(w.B, w.H, 128, device=DEV))


def test_graph_log_append_and_merge():
    """One whole cycle of M = 4 per block (three appends, then the merge)."""
    w = wl.custom(wl.WORKLOADS[5], B=2, H=5, M=4)
    C = w.M - 1
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    bufs = new_log_buffers(w, C)
    bufs["Sbase"] = S0.clone()
    ins = [dev_inputs(w, t)[1] for t in range(w.M)]

    def block(b, y):
        L = 0
        for d in ins:
            L = log_step(w, C, L, b["Sbase"], b, d, y)

    _check_rounds(block, _twin(bufs), _twin(bufs), torch.zeros(w.B, w.H, 128, device=DEV),
                  torch.zeros(w.B, w.H, 128, device=DEV))


@pytest.mark.parametrize("bits", [8, 4])
def test_graph_leapquant_window(bits):
    """One whole LeapQuant window of W = 4 per block, the boundary refit included."""
    m = rsu()
    w = wl.custom(wl.WORKLOADS[6] if bits == 8 else wl.WORKLOADS[12], B=2, H=5, W=4)
    bufs = new_lq_buffers(w)
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    quant, win = (m.gdn_lq_quantize, m.gdn_lq_window) if bits == 8 else (m.gdn_lq4_quantize, m.gdn_lq4_window)
    quant(S0, 4, bufs["Z"], bufs["B"], bufs["C"], bufs["Kc"], bufs["Uc"])
    ins = [dev_inputs(w, t)[1] for t in range(w.W)]

    def block(b, y):
        for t, d in enumerate(ins):
            win(w.W, t, 1, b["Z"], b["B"], b["C"], b["Kc"], b["Uc"], b["Kbuf"], b["Ubuf"], b["Gbuf"],
                d["q"], d["k"], d["v"], d["gate"], d["beta"], y)

    _check_rounds(block, _twin(bufs), _twin(bufs), torch.zeros(w.B, w.H, 128, device=DEV),
                  torch.zeros(w.B, w.H, 128, device=DEV))


def test_graph_stepq():
    """Four packed-state steps per block (decode, update, readout, repack)."""
    from parity import new_stepq_buffers
    m = rsu()
    w = wl.custom(wl.WORKLOADS[13], B=2, H=5)
    bufs = new_stepq_buffers(w)
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    om = torch.from_numpy(wl.row_influence(w)).to(DEV).view(w.B, w.H, 128)
    m.stepq_pack(S0, om, bufs["Z"], bufs["R"], bufs["C"])
    ins = [dev_inputs(w, t)[1] for t in range(4)]

    def block(b, y):
        for d in ins:
            m.gdn_stepq_step(b["Z"], b["R"], b["C"], om, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)

    _check_rounds(block, _twin(bufs), _twin(bufs), torch.zeros(w.B, w.H, 128, device=DEV),
                  torch.zeros(w.B, w.H, 128, device=DEV))
