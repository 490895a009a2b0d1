"""The decode step of a Llama-3-8B-shaped stack as the benchmark runs it: per
layer four group calls (q/k/v, o, gate/up, down) captured in one HIP graph,
replayed several times with the outputs poisoned in between, at 1 and 32
tokens and group sizes 128 and 64 (bjdmk.com.cn page "大模型量化技术极速优化…",
section "量化参数配置": group size is a parameter of the 4-bit format).  Two
layers; every output is checked against the float64 oracle on sampled
columns (packed weights from the oracle's pack), and every replay must give
the bits of the first."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
LAYERS = 2
ALPHA = {"q": 0.5, "k": 0.4, "v": 0.45, "o": 0.35, "gate": 0.4, "up": 0.3, "down": 0.45}


@pytest.fixture(scope="module")
def P():
    import weight_only_int4_awq_amd as P
    P.load()
    assert torch.cuda.is_available()
    return P


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _stack(g):
    """Per layer and linear: device (qweight, scales, qzeros, inv_s16), host pack, inv_s16."""
    layers = []
    for layer in range(LAYERS):
        row = {}
        for nm, n, k in S.LLAMA3_8B_LINEARS:
            w, x_cal, _, _ = S.config_layer(5, nm, n, k, 128, 0, 0.02, 0.01, 20.0, layer=layer)
            s16 = O.scale_candidate(O.calib_stats(x_cal), ALPHA[nm])
            inv = O.fp16_rn(1.0 / s16.astype(np.float64))
            hq, hs, hz, _ = O.pack_int4(w, s16, g)
            del w
            row[nm] = ((dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32)), dev(inv)), (hq, hs, hz), inv)
        layers.append(row)
    return layers


GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("g", [128, 64])
def test_stack_decode_graph_replays(P, g):
    stack = _stack(g)
    shapes = {nm: (n, k) for nm, n, k in S.LLAMA3_8B_LINEARS}
    for m in (1, 32):
        xs, ys = [], []
        for layer in range(LAYERS):
            xl = {}
            for inp, k in (("attn_in", 4096), ("o", 4096), ("mlp_in", 4096), ("down_in", 14336)):
                slot = S.SLOTS.get(inp)
                ch = S.outlier_channels(k, 0.01, S.seed_of(5, layer, slot, 3))
                xl[inp] = S.activations(m, k, S.seed_of(5, layer, slot, 2) + m, ch, 20.0)
            xs.append(xl)
            ys.append({nm: torch.empty((m, n), dtype=torch.float16, device=DEV) for nm, (n, k) in shapes.items()})
        xd = [{inp: dev(v) for inp, v in xl.items()} for xl in xs]
        # one workspace for the whole step: its calls are ordered on one stream
        need = max(P.awq_linear_group_workspace_size([shapes[nm][0] for nm in grp], m, shapes[grp[0]][1], g)
                   for grp in GROUPS)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)

        def step():
            for layer in range(LAYERS):
                for grp in GROUPS:
                    items = []
                    for nm in grp:
                        qw, sc, qz, inv = stack[layer][nm][0]
                        items.append((xd[layer][S.INPUT_OF[nm]], qw, sc, qz, inv, ys[layer][nm]))
                    P.awq_linear_w4a16_group(items, g=g, workspace=ws if need else None)

        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gr, stream=stream):
                step()
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        first = None
        for rep in range(3):
            for yl in ys:
                for y in yl.values():
                    y.fill_(float("nan"))
            gr.replay()
            torch.cuda.synchronize()
            cur = {(layer, nm): ys[layer][nm].clone() for layer in range(LAYERS) for nm in shapes}
            if first is None:
                first = cur
            else:
                for key, y in cur.items():
                    assert torch.equal(y.view(torch.int16), first[key].view(torch.int16)), (rep, key)
        rng = np.random.Generator(np.random.PCG64(990 + m + g))
        for layer in range(LAYERS):
            for nm, (n, k) in shapes.items():
                host, inv = stack[layer][nm][1], stack[layer][nm][2]
                cols = np.unique(np.concatenate([rng.choice(n, 64, replace=False), np.arange(n - 4, n)]))
                yr = O.linear_ref_rows(xs[layer][S.INPUT_OF[nm]], *host, inv, k, g, cols)
                got = first[(layer, nm)].cpu().numpy()[:, cols]
                ok, worst, raw = O.check_linear(got, yr)
                assert ok, (m, g, layer, nm, worst, raw)
