"""Planted mistakes in the CPU oracle must be caught by the pins.

Each mutation rewrites one line of one oracle function (a dropped term, a
wrong sign, index or operand, a missing rotation ...), swaps the rewritten
function into ``oracle.reference`` for the duration of the test, and runs the
pins of tests/pins.py until one fails.  A mutation that no pin notices would
mean the pins leave that part of the oracle unchecked.  Everything here runs
on the CPU and only touches the oracle.
"""
import inspect
import textwrap

import pytest

import oracle.reference as R
import pins

MUTATIONS = [
    # rotary embedding
    ("rope_neox", "y[..., :half] = x1 * c - x2 * s", "y[..., :half] = x1 * c + x2 * s"),
    ("rope_neox", "y[..., half:] = x2 * c + x1 * s", "y[..., half:] = x2 * c - x1 * s"),
    ("rope_neox", "x1 = x[..., :half]\n    x2 = x[..., half:]",
     "x1 = x[..., 0::2]\n    x2 = x[..., 1::2]"),                         # interleaved pairs
    ("rope_neox", "np.asarray(positions, dtype=np.float64)[:, None]",
     "(np.asarray(positions, dtype=np.float64) + 1)[:, None]"),             # position off by one
    ("rope_neox", "c = np.cos(a)[:, None, :]", "c = np.cos(a)[:, None, :] * 0 + 1"),  # dropped cos
    ("rope_inv_freq", "-2.0 * i / float(head_dim)", "-1.0 * i / float(head_dim)"),
    ("rope_inv_freq", "np.power(float(theta),", "np.power(10000.0,"),      # base ignored
    # dynamic-NTK rope scaling
    ("rope_dynamic_ntk", "** (d / (d - 2.0))", "** (d / (d - 1.0))"),       # wrong exponent
    ("rope_dynamic_ntk", "(s * L / float(original_max_position) - (s - 1.0))",
     "(s * L / float(original_max_position))"),                            # (factor - 1) dropped
    ("rope_dynamic_ntk", "L = int(s * int(original_max_position))", "L = int(original_max_position)"),
    # rounding
    ("f64_to_bf16_bits", "r = np.rint(xf / ulp) * ulp", "r = np.trunc(xf / ulp) * ulp"),
    ("f64_to_bf16_bits", "r = np.rint(xf / ulp) * ulp",
     "xf = xf.astype(np.float32).astype(np.float64)\n    r = np.rint(xf / ulp) * ulp"),  # double rounding
    # cache write / gather
    ("rope_cache_write", "blk, off = divmod(slot, B)", "off, blk = divmod(slot, B)"),
    ("rope_cache_write", "v_store = heads[:, H + Hkv:]",
     "v_store = from_f64(rope_neox(x[:, H + Hkv:], positions, theta), dtype)"),  # v rotated
    ("rope_cache_write", "k_rot = rope_neox(xk, positions, theta)",
     "k_rot = xk"),                                                         # k not rotated
    ("rope_cache_write", "xq, xk = x[:, :H], x[:, H:H + Hkv]",
     "xq, xk = x[:, :H], x[:, H + Hkv:]"),                                  # k from v columns
    ("gather_kv", "off = j % B", "off = (j + 1) % B"),
    ("gather_kv", "V = to_f64(np.asarray(v_cache)[blk, :, :, off], dtype)",
     "V = to_f64(np.asarray(v_cache)[blk, :, off % np.asarray(v_cache).shape[2], :], dtype)"),
    # attention
    ("causal_visible", "<= pq[:, None]", "< pq[:, None]"),
    ("causal_visible", "pq = c - n + np.arange(n)", "pq = np.arange(n)"),   # top-left alignment
    ("softmax_rows", "return w / w.sum(axis=-1, keepdims=True)", "return w"),
    ("softmax_rows", "np.exp(zm - m)", "np.exp(2.0 * (zm - m))"),
    ("kv_head_for", "h // (num_heads // num_kv_heads)", "h % num_kv_heads"),
    ("default_scale", "float(head_dim) ** -0.5", "float(head_dim) ** -1.0"),
    ("attention_varlen", "out[r0:r1, h, :] = pi @ V[:, g, :]", "out[r0:r1, h, :] = pi @ K[:, g, :]"),
    ("attention_varlen", "z = scale * (qf[r0:r1, h, :] @ K[:, g, :].T)",
     "z = scale * (qf[r0:r1, h, :] @ V[:, g, :].T)"),
    ("attention_varlen", "n, c = r1 - r0, int(context_lens[s])", "n, c = r1 - r0, int(context_lens[s]) - 1"),
    # shared-prefix cascade
    ("attention_decode_cascade", "Ks, Vs = K[L:], V[L:]", "Ks, Vs = K, V"),        # prefix counted twice
    ("attention_decode_cascade", "Ks, Vs = K[L:], V[L:]", "Ks, Vs = K[L + 1:], V[L + 1:]"),
    ("attention_decode_cascade", "/ (l1 * e1 + l2 * e2)", "/ (l1 + l2)"),         # normalisers not rescaled
    ("attention_decode_cascade", "e1, e2 = np.exp(m1 - M), np.exp(m2 - M)",
     "e1, e2 = np.exp(M - m1), np.exp(M - m2)"),
    ("attention_decode_cascade", "m1, l1, a1 = _partial_state(qf[s, h],",
     "m1, l1, a1 = _partial_state(qf[members[0], h],"),                         # first member's q
    ("_partial_state", "w = np.exp(z - m)", "w = np.exp(z - 2 * m)"),
    ("check_prefix_groups", "if not np.array_equal(np.asarray(block_tables[s])[:L // B], ids):",
     "if False:"),
    # Qwen3 q/k norm
    ("rms_norm_heads", "np.sqrt(ms + float(eps))", "np.sqrt(ms)"),          # eps dropped
    ("rms_norm_heads", "ms = np.mean(x * x, axis=-1, keepdims=True)",
     "ms = np.sum(x * x, axis=-1, keepdims=True)"),                         # sum, not mean
    ("rms_norm_heads", "* np.asarray(weight, dtype=np.float64)", "* 1.0"),  # weight ignored
    ("rope_cache_write", "xq = rms_norm_heads(xq, to_f64(q_norm_weight, dtype), rms_eps)",
     "xq = rms_norm_heads(xq, to_f64(k_norm_weight, dtype), rms_eps)"),     # weights swapped
    # FP8 cache codes and scales
    ("fp8_e4m3_decode", "(1.0 + m / 8.0)", "(m / 8.0)"),                  # implicit one dropped
    ("fp8_e4m3_decode", "np.exp2((e - 7)", "np.exp2((e - 8)"),            # wrong bias
    ("fp8_e4m3_encode", "m = np.rint((frac - 1.0) * 8.0)", "m = np.floor((frac - 1.0) * 8.0)"),
    ("fp8_e4m3_encode", "a = np.minimum(np.abs(x), E4M3_MAX)", "a = np.abs(x)"),   # no saturation
    ("fp8_e4m3_encode", "np.rint(a[sub] / 2.0 ** -9)", "np.rint(a[sub] / 2.0 ** -10)"),
    ("rope_cache_write", "k_store = fp8_e4m3_encode(k_rot / float(k_scale))",
     "k_store = fp8_e4m3_encode(k_rot * float(k_scale))"),
    ("rope_cache_write", "v_store = fp8_e4m3_encode(x[:, H + Hkv:] / float(v_scale))",
     "v_store = fp8_e4m3_encode(x[:, H + Hkv:] / float(k_scale))"),
    ("gather_kv", "V = value[np.asarray(v_cache)[blk, :, :, off]] * float(v_scale)",
     "V = value[np.asarray(v_cache)[blk, :, :, off]] * float(k_scale)"),
]


def _mutant(fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(R, fname)))
    assert old in src, (fname, old)
    ns = dict(vars(R))
    exec(compile(src.replace(old, new, 1), f"<mutant {fname}>", "exec"), ns)
    return ns[fname]


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_mutation_is_caught(monkeypatch, fname, old, new):
    monkeypatch.setattr(R, fname, _mutant(fname, old, new))
    for pin in pins.ALL_PINS:
        try:
            pin(R)
        except Exception:
            return
    pytest.fail(f"no pin caught the mutation in {fname}: {new!r}")
