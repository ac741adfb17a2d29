"""Plants plausible mistakes in a temporary copy of the oracle and checks
that the pins catch every one (CPU only; the real oracle is never edited).

The committed golden sample was written by the oracle itself, so it is not
an independent pin: the copies run every pin except that regression check,
and an unmutated copy must pass them all (otherwise every mutant would look
caught)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "eps_outside_root": ("np.sqrt(ms + eps)", "(np.sqrt(ms) + eps)"),
    "gain_offset": ("return x / np.sqrt(ms + eps) * _f64(gain)",
                    "return x / np.sqrt(ms + eps) * (1 + _f64(gain))"),
    "rope_sin_sign": ("x[..., : rd // 2] = a * cos - b * sin",
                      "x[..., : rd // 2] = a * cos + b * sin"),
    "rope_freq_exponent": ("inv_freq = theta ** (-2.0 * i / rot_dim)",
                           "inv_freq = theta ** (-1.0 * i / rot_dim)"),
    "rope_position_off_by_one": ("positions = start_pos + np.arange(B)",
                                 "positions = start_pos + 1 + np.arange(B)"),
    "gqa_map_modulo": ("return h // (n_heads // n_kv_heads)", "return h % n_kv_heads"),
    "causal_leaks_next_key": ("visible = np.arange(T)[None, :] <= pos",
                              "visible = np.arange(T)[None, :] <= pos + 1"),
    "softcap_before_scale": (
        "s = (q[:, h, :] @ k_all[:, g, :].T) * scale\n        if softcap:\n"
        "            s = softcap * np.tanh(s / softcap)",
        "s = (q[:, h, :] @ k_all[:, g, :].T)\n        if softcap:\n"
        "            s = softcap * np.tanh(s / softcap)\n        s = s * scale"),
    "gate_dropped": ("o = o * (1.0 / (1.0 + np.exp(-_f64(gate))))", "o = o"),
    "gate_interleaved": ("q, gate = qg[:, : Hq * hd], None", "q, gate = qg[:, 0::2], None"),
    "k_bias_dropped": ("q, k, v = q + _f64(w[\"bq\"]), k + _f64(w[\"bk\"]), v + _f64(w[\"bv\"])",
                       "q, k, v = q + _f64(w[\"bq\"]), k, v + _f64(w[\"bv\"])"),
    "qk_norm_dropped": ("        q = rms_norm(q, w[\"q_norm\"], spec.rms_eps)\n"
                        "        k = rms_norm(k, w[\"k_norm\"], spec.rms_eps)\n",
                        "        pass\n"),
    "attn_residual_dropped": ("    x1 = x + attn\n", "    x1 = 0 * x + attn\n"),
    "wo_transposed": ("attn = o.reshape(B, -1) @ _f64(w[\"wo\"]).T",
                      "attn = o.reshape(B, -1) @ _f64(w[\"wo\"]).reshape("
                      "_f64(w[\"wo\"]).shape[::-1])"),
    "ffn_norm_reads_x": ("h2 = rms_norm(x1, w[\"g_ffn\"]", "h2 = rms_norm(x, w[\"g_ffn\"]"),
    "silu_as_sigmoid": ("return z / (1.0 + np.exp(-z))", "return 1 / (1.0 + np.exp(-z))"),
    "prefix_v_reads_k": ("v_all = np.concatenate([_f64(prefix_v)",
                         "v_all = np.concatenate([_f64(prefix_k)"),
    "window_off_by_one": ("visible &= np.arange(T)[None, :] > pos - window",
                          "visible &= np.arange(T)[None, :] >= pos - window"),
    "mscale_on_every_channel": ("x[..., :rd] *= mscale", "x *= mscale"),
    "freq_factor_multiplies": ("inv_freq = inv_freq / _f64(freq_factors)",
                               "inv_freq = inv_freq * _f64(freq_factors)"),
    "rope_options_dropped": ("freq_factors=getattr(spec, \"rope_freq_factors\", None),",
                             "freq_factors=None,"),
    "gelu_tanh_form": ("return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))",
                       "return 0.5 * z * (1.0 + np.tanh(0.7978845608 * (z + 0.044715 * z ** 3)))"),
    "geglu_runs_silu": ("a = gelu(g) if act == \"geglu\" else silu(g)", "a = silu(g)"),
    "post_attn_norm_after_residual": ("    x1 = x + attn\n",
                                      "    x1 = x + attn\n    if \"g_post_attn\" in w:\n"
                                      "        x1 = rms_norm(x + o.reshape(B, -1) @ _f64(w[\"wo\"]).T, "
                                      "w[\"g_post_attn\"], spec.rms_eps)\n"),
    "post_ffn_norm_dropped": ("        ffn = rms_norm(ffn, w[\"g_post_ffn\"], spec.rms_eps)", "        pass"),
    "stack_unchained": ("x, k, v = dense_layer(x, w, spec, start_pos, pk, pv)",
                        "_, k, v = dense_layer(_f64(hidden), w, spec, start_pos, pk, pv)\n"
                        "        x = _"),
    "stack_rows_reversed": ("    return x, ks, vs\n", "    return x, ks[::-1], vs[::-1]\n"),
    "stack_rows_of_first_layer": ("        ks.append(k)\n", "        ks.append(ks[0] if ks else k)\n"),
    "decode_skips_new_row": ("k_all = np.concatenate([_f64(cache_k)[:rows], _f64(k)[None]])",
                             "k_all = np.concatenate([_f64(cache_k)[:rows], "
                             "_f64(cache_k)[rows - 1:rows]])"),
}


@pytest.fixture(scope="module")
def oracle_source():
    with open(os.path.join(ROOT, "oracle", "__init__.py")) as f:
        return f.read()


def run_pins(tmp_path, source):
    """Runs the independent pins against a copy of the oracle holding `source`."""
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "golden"))
    (tmp_path / "oracle" / "__init__.py").write_text(source)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-k", "not committed_sample", "tests/test_oracle_pins.py"],
                          cwd=tmp_path, capture_output=True, text=True, timeout=300)


def test_unmutated_copy_passes_the_pins(oracle_source, tmp_path):
    r = run_pins(tmp_path, oracle_source)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, oracle_source, tmp_path):
    before, after = MUTANTS[name]
    assert before in oracle_source, f"mutation site of {name} not found"
    r = run_pins(tmp_path, oracle_source.replace(before, after))
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"
