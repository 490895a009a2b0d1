"""GPU scale search on whole layers at the workloads' own sizes against the
float64 oracle: the chosen alpha index, s16 and inv_s16 bit for bit, every loss
within the bound derived from the kernel's arithmetic (tests/search_bound.py).
The search picks the alpha that minimises the quantized layer's output error
(jsqmd.com page "从Java转行大模型应用，大模型量化实现，AWQ 与 GPTQ 算法",
section 二.1 (3)).  Each case prints the oracle's best-vs-second gap and its
margin over the two losses' bounds (run with -rA to see them).

* the single 4096 x 4096 linear with 128 calibration tokens (N(0, 0.02)
  weights, 1 % of the channels x20), whole layer;
* the Llama-3-8B-shaped k and v projections (1024 x 4096) with 512
  calibration tokens, whole layers;
* the Llama-3-70B-shaped linears (N(0, 0.015) weights, 0.5 % of the channels
  x30, 128 calibration tokens) at full K on sampled rows: the loss is a sum
  over rows, so this is the search of those rows.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O
from tests import search_bound as SB

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def P():
    import weight_only_int4_awq_amd as P
    P.load()
    assert torch.cuda.is_available()
    return P


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _search_vs_oracle(P, w, x, g, n_grid, label):
    wd, xd = dev(w), dev(x)
    a_dev = P.awq_calib_stats(xd)
    ws = torch.empty(P.awq_search_workspace_size(w.shape[0], w.shape[1], x.shape[0], g, n_grid),
                     dtype=torch.uint8, device=DEV)
    best, s16, inv, losses = P.awq_search_scale(wd, xd, a_dev, g=g, n_grid=n_grid, workspace=ws)
    torch.cuda.synchronize()
    a = O.calib_stats(x)
    assert np.array_equal(a_dev.cpu().numpy().view(np.uint64), a.view(np.uint64))
    ob, os16, oinv, olosses = O.search_scale(w, x, a, g=g, n_grid=n_grid)
    dnorm = SB.loss_bounds(w, x, a, g, n_grid)
    worst = SB.check_losses(losses.cpu().numpy(), olosses, dnorm)
    b, second, gap, margin = SB.gap_report(olosses, dnorm)
    print(f"search gap [{label}]: best {ob} (alpha {ob / n_grid:.2f}) second {second} gap {gap:.3e} "
          f"margin {margin:.3g} max rel loss err {worst:.2e} L_best/L_0 {olosses[ob] / olosses[0]:.4f}")
    assert int(best.item()) == ob, (int(best.item()), ob, gap, margin)
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), os16.view(np.uint16))
    assert np.array_equal(inv.cpu().numpy().view(np.uint16), oinv.view(np.uint16))
    assert olosses[ob] < olosses[0]          # the outlier channels make scaling pay
    return ob, gap, margin


@pytest.mark.timeout(900)
def test_search_single_linear_4096_whole_layer(P):
    w, x_cal, _, _ = S.config_layer(1, "q", 4096, 4096, 128, 0, 0.02, 0.01, 20.0)
    _search_vs_oracle(P, w, x_cal, 128, 20, "4096x4096, 128 tokens")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["k", "v"])
def test_search_llama3_8b_kv_whole_layer_512_tokens(P, name):
    w, x_cal, _, _ = S.config_layer(3, name, 1024, 4096, 512, 0, 0.02, 0.01, 20.0)
    _search_vs_oracle(P, w, x_cal, 128, 20, f"llama3-8b {name} 1024x4096, 512 tokens")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n,k", S.LLAMA3_70B_LINEARS)
def test_search_llama3_70b_sampled_rows(P, name, n, k):
    w, x_cal, _, _ = S.config_layer(4, name, n, k, 128, 0, 0.015, 0.005, 30.0)
    rows = np.sort(np.random.Generator(np.random.PCG64(n + k)).choice(n, 96, replace=False))
    _search_vs_oracle(P, np.ascontiguousarray(w[rows]), x_cal, 128, 20,
                      f"llama3-70b {name} {n}x{k} (96 rows), 128 tokens")
