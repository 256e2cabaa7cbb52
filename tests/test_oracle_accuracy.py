"""The accuracy soft report (not a parity gate): on every benchmark
configuration's synthetic activations, the relative error of the SharQ
two-path product, ||Y - X W^T|| / ||X W^T|| against the unquantised fp64
product, next to the same quantity for plain MXFP4 activations against the
same MXFP4 weights. This is the synthetic stand-in for the pages' accuracy
story (SharQ page, Abstract: the decomposition recovers most of the FP4 loss);
real weights and zero-shot suites are not available here. The one property
asserted is that the decomposition is more accurate than plain MXFP4 on every
configuration. Run with -s to see the table."""

import numpy as np
import pytest

from oracle import (absorb_gamma, linear_ref, mxfp4_dequantize, mxfp4_quantize, prepare_ref,
                    quantize_weight_ref, unpack_nibbles)
from synth import (normal_weight, workload_down_silu, workload_linear, workload_llama70b_decode,
                   workload_llama8b_mlp, workload_qwen3_moe)

ROWS, OUTS = 64, 256


def _case(name):
    rng = np.random.default_rng(77)
    if name == "c1 linear 128x4096, 2:4":
        x, g, n, m = workload_linear()["x"][:ROWS], None, 2, 4
    elif name == "c2 llama8b x (gamma), 2:4":
        wl = workload_llama8b_mlp(with_weights=False)
        x, g, n, m = wl["x"][:ROWS], wl["gamma"], 2, 4
    elif name.startswith("c3"):
        x = workload_down_silu(with_weights=False)["x"][:ROWS]
        g = None
        n, m = (8, 16) if "8:16" in name else (2, 4)
    elif name == "c4 llama70b decode T=8, 2:4":
        x, g, n, m = workload_llama70b_decode(8, with_weights=False)["x"], None, 2, 4
    else:
        x, g, n, m = workload_qwen3_moe(with_weights=False)["x"][:ROWS], None, 2, 4
    w = normal_weight(rng, OUTS, x.shape[1])
    return x, g, w, n, m


@pytest.mark.parametrize("name", ["c1 linear 128x4096, 2:4", "c2 llama8b x (gamma), 2:4", "c3 down input, 8:16",
                                  "c3 down input, 2:4", "c4 llama70b decode T=8, 2:4", "c5 qwen3 tokens, 2:4"])
def test_decomposition_beats_plain_mxfp4(name):
    x, g, w, n, m = _case(name)
    xp = absorb_gamma(x, g).astype(np.float64)
    w_exact = absorb_gamma(w, None).astype(np.float64)
    y_exact = xp @ w_exact.T
    wc, ws = quantize_weight_ref(w)
    p = prepare_ref(x, g, n, m)
    y_sharq, _ = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    c, e = mxfp4_quantize(absorb_gamma(x, g))
    w_deq = mxfp4_dequantize(unpack_nibbles(wc), ws.astype(np.int64) - 127)
    y_mx = mxfp4_dequantize(c, e) @ w_deq.T
    y_wq = xp @ w_deq.T  # activations exact, weights MXFP4: the floor set by the weight quantisation
    norm = np.linalg.norm(y_exact)
    err_sharq = np.linalg.norm(y_sharq - y_exact) / norm
    err_mx = np.linalg.norm(y_mx - y_exact) / norm
    err_w = np.linalg.norm(y_wq - y_exact) / norm
    print(f"\n  {name}: SharQ {err_sharq:.4f}  plain MXFP4 {err_mx:.4f}  weights-only floor {err_w:.4f}")
    assert err_sharq < err_mx
