"""Why the decode path has no fp8-MFMA variant (queries or softmax weights in
e4m3 so that the products run at the fp8 matrix rate): on the oracle, with
the fp8 operand scaled per row to the e4m3 range (max 448) and rounded to
nearest, the output misses the parity bar (relative L2 <= 5e-3) by a factor
of four or more.  A split of each bf16 operand into two e4m3 parts would be
exact but needs two fp8 products per bf16 product, which is no faster.  CPU
only; the numbers are printed."""
import numpy as np

from oracle import reference_decode
from oracle.codecs import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode_satfinite
from oracle.mla_oracle import absorb_query, out_projection, sequence_rows, softmax_with_lse
from workload import configs, make_inputs

BAR = 5e-3


def _e4m3_rows(x):
    """Each row scaled to the e4m3 range, rounded to e4m3, scaled back."""
    s = np.max(np.abs(x), axis=-1, keepdims=True) / 448.0
    s = np.where(s == 0, 1.0, s)
    return e4m3fn_decode(e4m3fn_encode_satfinite((x / s).astype(np.float32))) * s


def test_e4m3_queries_or_weights_miss_the_bar():
    wl = configs.V3.with_(name="v3_fp8mfma", batch=2, seq_len=None, seq_lens=(1024, 333))
    inp = make_inputs(wl)
    ref = reference_decode(inp)["out"]
    w_uk, w_uv = bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)
    errs = {}
    for mode in ("q", "p"):
        outs = []
        for b in range(wl.batch):
            q = absorb_query(bf16_bits_to_f64(inp.q_nope[b]), bf16_bits_to_f64(inp.q_pe[b]), w_uk,
                             int(inp.seq_lens[b]) - 1, wl.rope_base)
            C, Kr = sequence_rows(inp, b)
            if mode == "q":
                q = _e4m3_rows(q)
            p, _ = softmax_with_lse(wl.softmax_scale * (q @ np.concatenate([C, Kr], -1).T))
            if mode == "p":
                p = _e4m3_rows(p)
            outs.append(out_projection(p @ C, w_uv))
        x = np.stack(outs)
        errs[mode] = float(np.linalg.norm(x - ref) / np.linalg.norm(ref))
        print(f"e4m3 {mode}: rel L2 of out = {errs[mode]:.3e} (bar {BAR:g})")
    assert errs["q"] > 4 * BAR and errs["p"] > 3 * BAR
