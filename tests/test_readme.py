"""The README's usage example runs as written, and its description of the
output layout holds: layer l keeps lengths[(l // n_reuse) * H_kv + h] rows of
head h at rows h * L_cap .. of its compacted K/V."""
import os
import re

import pytest

torch = pytest.importorskip("torch")

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _example() -> str:
    text = open(README).read()
    m = re.search(r"## Usage \(Python binding\)\s*```python\n(.*?)```", text, re.S)
    assert m, "README has no Python usage block"
    return m.group(1)


def test_readme_example_parses():
    compile(_example(), "README.md", "exec")


@pytest.mark.gpu
def test_readme_example_runs_and_layout_holds():
    ns = {}
    exec(compile(_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    ck, prob, buf = ns["ck"], ns["prob"], ns["buf"]
    k, v, Hkv, n_reuse, n_layers = ns["k"], ns["v"], ns["Hkv"], ns["n_reuse"], ns["n_layers"]
    l_cap = ck.plan(prob)["l_cap"][0]
    lengths = buf.lengths.cpu()
    indices = buf.indices.cpu()
    per_anchor = indices.numel() // buf.n_anchor
    for l in (0, 1, n_layers - 1):
        a = l // n_reuse
        for h in (0, Hkv - 1):
            n = int(lengths[a * Hkv + h])
            assert 0 < n <= l_cap
            idx = indices[a * per_anchor + h * l_cap: a * per_anchor + h * l_cap + n].long().to("cuda")
            assert torch.equal(buf.k_out[l][h * l_cap: h * l_cap + n], k[l][idx, h])
            assert torch.equal(buf.v_out[l][h * l_cap: h * l_cap + n], v[l][idx, h])
            kk, vv, pos = buf.kept(l, 0, h)
            assert torch.equal(pos.long(), idx) and torch.equal(kk, k[l][idx, h]) and torch.equal(vv, v[l][idx, h])
    kk, vv, pos = ns["k_kept"], ns["v_kept"], ns["positions"]
    assert kk.shape[0] == vv.shape[0] == pos.numel() > 0
