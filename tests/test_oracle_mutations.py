"""The oracle's pins have teeth: each plausible mistake, planted in a
temporary copy of the oracle's C source (on the CPU, never on a GPU), must
make ``tests/test_oracle.py`` fail.

Mistakes covered: dropped 1/sqrt(d) (Kara eq. 1), flipped exponent sign,
interleaved GQA head mapping, wrong observe-window rows (Algorithm 1 step 1),
off-by-one chunk bounds (step 3), averaged short last chunk, causal masking,
reversed tie order and ascending sort in TopK (step 4), a short recent window
(step 5), gathering the wrong head (step 6), reused layers gathering the
anchor layer's cache (Algorithm 2), a bad bf16 widening and swapped key
strides; in the decode-attention consumer, a dropped 1/sqrt(d), a flipped
exponent sign, values taken from the keys and every query head reading the
first query; in the paged layout (Python), pages chosen by i mod P, rows by
i div P, negative page ids kept and rows shifted by one.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "chunkkv_oracle.c")

MUTATIONS = {
    "drop_scale": ("const double inv_sqrt_d = 1.0 / sqrt((double)d);", "const double inv_sqrt_d = 1.0;"),
    "exp_sign": ("scores[t / c] += exp(x[t] - m) / s;", "scores[t / c] += exp(m - x[t]) / s;"),
    "gqa_interleave": ("const int hq = h * G + g;", "const int hq = h + g * n_kv_heads;"),
    "first_rows": ("const int64_t qt = t_q - w + r;", "const int64_t qt = r;"),
    "chunk_off_by_one": ("scores[t / c] +=", "scores[(t + 1) / c < C ? (t + 1) / c : C - 1] +="),
    "avg_last_chunk": ("  free(x);\n  return ORC_OK;",
                       "  scores[C - 1] /= (double)(T - (C - 1) * c);\n  free(x);\n  return ORC_OK;"),
    "causal_mask": ("for (int64_t t = 0; t < T; ++t) s += exp(x[t] - m);",
                    "for (int64_t t = 0; t <= qt && t < T; ++t) s += exp(x[t] - m);"),
    "tie_high_id_first": ("return (x->id > y->id) - (x->id < y->id);", "return (x->id < y->id) - (x->id > y->id);"),
    "topk_ascending": ("if (x->score > y->score) return -1;", "if (x->score < y->score) return -1;"),
    "short_window": ("for (int64_t t = T - w; t < T; ++t) keep[t] = 1;",
                     "for (int64_t t = T - w + 1; t < T; ++t) keep[t] = 1;"),
    "gather_head0": ("(int64_t)head * head_stride) * elem_bytes", "(int64_t)0 * head_stride) * elem_bytes"),
    "reuse_anchor_cache": ("orc_gather(n, idx, eb, d, k[l],", "orc_gather(n, idx, eb, d, k[anchor],"),
    "bf16_shift": ("<< 16;", "<< 15;"),
    "decode_drop_scale": ("x[i] = acc * inv_sqrt_d;", "x[i] = acc;"),
    "decode_exp_sign": ("const double p = exp(x[i] - m) / s;", "const double p = exp(m - x[i]) / s;"),
    "decode_values_from_keys": ("+= p * widen(v, dtype, i * d + j);", "+= p * widen(k, dtype, i * d + j);"),
    "decode_query_head0": ("widen(q, dtype, (int64_t)g * d + j)", "widen(q, dtype, (int64_t)0 * d + j)"),
    "k_strides_swapped": ("widen(k, dtype, t * k_tok_stride + (int64_t)h * k_head_stride + i)",
                          "widen(k, dtype, t * k_head_stride + (int64_t)h * k_tok_stride + i)"),
}


def _run(name, tmp):
    a, b = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(a) >= 1, name
    c_path = os.path.join(tmp, name + ".c")
    so_path = os.path.join(tmp, name + ".so")
    open(c_path, "w").write(src.replace(a, b, 1))   # the first occurrence: the function the mistake names
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-o", so_path, c_path, "-lm"])
    env = dict(os.environ, CHUNKKV_ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda n: _run(n, tmp), MUTATIONS))
    missed = [n for n, rc in results if rc == 0]
    assert not missed, f"pins did not catch: {missed}"


# The paged layout is Python: each mistake is planted in a copy of
# oracle.to_pages compiled in memory, and the page pins of test_oracle.py are
# run against it in this process.
PAGE_MUTATIONS = {
    "page_by_mod": ("page = int(table[i // page_rows])", "page = int(table[i % page_rows])"),
    "row_by_div": ("pool[page, i % page_rows]", "pool[page, i // page_rows]"),
    "keeps_negative_ids": ("if 0 <= page < n_pages:", "if page < n_pages:"),
    "shifted_rows": ("= rows[i]", "= rows[max(i - 1, 0)]"),
}


def _page_pins():
    import test_oracle as t
    yield t.test_to_pages_worked_example
    yield t.test_to_pages_one_large_page_is_the_contiguous_layout
    for n, p in ((97, 16), (250, 7)):
        yield lambda n=n, p=p: t.test_to_pages_read_back_through_the_table(n, p)
    yield t.test_to_pages_skips_out_of_range_page_ids


@pytest.mark.parametrize("name", sorted(PAGE_MUTATIONS))
def test_every_planted_page_layout_mistake_is_caught(name, monkeypatch):
    import inspect
    import textwrap

    import numpy as np

    import oracle
    src = textwrap.dedent(inspect.getsource(oracle.to_pages))
    a, b = PAGE_MUTATIONS[name]
    assert src.count(a) == 1, name
    ns = {"np": np}
    exec(compile(src.replace(a, b), f"<mutant {name}>", "exec"), ns)
    monkeypatch.setattr(oracle, "to_pages", ns["to_pages"])
    caught = False
    for pin in _page_pins():
        try:
            pin()
        except Exception:   # a failed assertion or an out-of-range write both count
            caught = True
            break
    assert caught, f"mutation {name} passed every page pin"
