"""Plants plausible mistakes in a private copy of the oracle and checks that
the pins catch each one (at least one pin fails).  CPU only; the real oracle
module is never modified."""
import inspect
import sys
import types

import pytest

from oracle import dspine_oracle as O
from tests import test_oracle_pins as P

MUTATIONS = {
    "rmsnorm eps outside sqrt": (
        "np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
        "(np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)"),
    "rmsnorm drops gain": (
        "return widen(w) * x / np.sqrt", "return x / np.sqrt"),
    "rope sign flipped": (
        "[x1 * cos - x2 * sin, x2 * cos + x1 * sin]", "[x1 * cos + x2 * sin, x2 * cos - x1 * sin]"),
    "rope halves swapped": (
        "[x1 * cos - x2 * sin, x2 * cos + x1 * sin]", "[x2 * cos + x1 * sin, x1 * cos - x2 * sin]"),
    "rope frequency exponent": (
        "np.power(float(theta), -2.0 * j / head_dim)", "np.power(float(theta), -1.0 * j / head_dim)"),
    "bridge uses own code for message": (
        "cp = c[t - 1] if pred_codes is None else pred_codes[t]",
        "cp = c[t] if pred_codes is None else pred_codes[t]"),
    "bridge drops rho scale": (
        "return x_t + rho_t * linear(", "return x_t + linear("),
    "bridge drops receiver gate term": (
        "gate = sigmoid(linear(c_t[None], wts[\"bridge_G\"])[0]\n                   + ",
        "gate = sigmoid(0 * linear(c_t[None], wts[\"bridge_G\"])[0]\n                   + "),
    "bridge drops bias": (
        "[0] + widen(wts[\"bridge_b\"]))", "[0])"),
    "bridge code without sqrt(r)": (
        "c = math.sqrt(r) * z / (np.linalg.norm", "c = z / (np.linalg.norm"),
    "bridge anchor code from wrong row": (
        "widen(wts[\"codebook\"][anchor_id])", "widen(wts[\"codebook\"][anchor_id - 1])"),
    "bridge writes anchor row": (
        "for t in range(1, W):\n        cp", "for t in range(0, W):\n        cp"),
    "swiglu operands swapped": (
        "silu(linear(m, wts[p + \"w_gate\"])) * linear(m, wts[p + \"w_up\"])",
        "silu(linear(m, wts[p + \"w_up\"])) * linear(m, wts[p + \"w_gate\"])"),
    "attention residual dropped": (
        "    y = x + o\n", "    y = o\n"),
    "post norm uses input gain": (
        "m = plain_rmsnorm(y, wts[p + \"g_post\"], g.eps)", "m = plain_rmsnorm(y, wts[p + \"g_in\"], g.eps)"),
    "window off by one": (
        "allowed &= np.abs(key_pos[None, :] - qpos) < S", "allowed &= np.abs(key_pos[None, :] - qpos) <= S"),
    "window predicate off by one": (
        "if window > 0 and abs(p_key - p_query) >= window:", "if window > 0 and abs(p_key - p_query) > window:"),
    "interval off by one": (
        "lo = max(0, frontier + row - window + 1)", "lo = max(0, frontier + row - window)"),
    "gqa head mapping modulo": (
        "        kvh = h // grp\n        s = qh", "        kvh = h % g.n_kv_heads\n        s = qh"),
    "attention scale missing": (
        "s = qh[:, h, :] @ K[:, kvh, :].T / math.sqrt(D)", "s = qh[:, h, :] @ K[:, kvh, :].T"),
    "ring keeps one extra position": (
        "    return max(0, frontier - window)\n", "    return max(0, frontier - window - 1)\n"),
    "v stored without bf16 step": (
        "v = round_fp16(round_bf16(v))", "v = round_fp16(v)"),
    "context norm gain dropped": (
        "return plain_rmsnorm(u, wts[\"g_ctx\"], g.eps)", "return plain_rmsnorm(u, np.ones(u.shape[-1]), g.eps)"),
    "block input shifted": (
        "rows = [anchor_id] + [g.mask_token_id] * (W - 1)", "rows = [g.mask_token_id] * W"),
    "bridge parameter count misses b": (
        "+ 3 * msg_dim * code_dim + msg_dim", "+ 3 * msg_dim * code_dim"),
    "bf16 rounding truncates": (
        "rounded = (bits + half - np.uint64(1) + lsb) >> drop << drop", "rounded = bits >> drop << drop"),
    "top-k ties prefer the larger id": (
        "order = np.lexsort((np.arange(scores.shape[0]), -scores))",
        "order = np.lexsort((-np.arange(scores.shape[0]), -scores))"),
    "top-k keeps the smallest scores": (
        "order = np.lexsort((np.arange(scores.shape[0]), -scores))",
        "order = np.lexsort((np.arange(scores.shape[0]), scores))"),
    "refinement ignores the candidate code": (
        "sr * widen(wts[\"codebook\"][s])", "c[t - 1]"),
    "refinement conditions row 1 on candidates": (
        "preds = [anchor_id] * K if t == 1 else", "preds = [int(v) for v in cand[0]] if t == 1 else"),
    "refinement predecessor from its own row": (
        "else [int(v) for v in cand[t - 2]]", "else [int(v) for v in cand[t - 1]]"),
    "table scores without the final norm": (
        "h = plain_rmsnorm(x, wts[\"g_final\"], g.eps)", "h = x"),
    "table scores the previous row's candidates": (
        "head_scores(lm_head, h, cand[t - 1])", "head_scores(lm_head, h, cand[max(t - 2, 0)])"),
    "greedy walk ignores the previous choice": (
        "choice[t] = int(np.argmax(T[t, i]))", "choice[t] = int(np.argmax(T[t, 0]))"),
    "greedy walk takes the last maximum": (
        "choice[t] = int(np.argmax(T[t, i]))", "choice[t] = int(len(T[t, i]) - 1 - np.argmax(T[t, i][::-1]))"),
    "sampled walk ignores temperature": (
        "s = np.asarray(T[t, i], dtype=np.float64) / float(temperature)",
        "s = np.asarray(T[t, i], dtype=np.float64)"),
    "sampled walk inclusive cdf": (
        "if float(uniforms[t]) < cdf:", "if float(uniforms[t]) <= cdf:"),
    "sampled walk keeps the wrong probability": (
        "q[t] = p[j]", "q[t] = p[i]"),
    "fp8 rounding truncates": (
        "return np.copysign(np.round(a / step) * step, x)", "return np.copysign(np.floor(a / step) * step, x)"),
    "fp8 subnormal step halved": (
        "e = np.maximum(ex - 1, -6)", "e = np.maximum(ex - 1, -7)"),
    "fp8 scale one power of two too small": (
        "sv[nz] = np.where(mant == 0.5, np.ldexp(1.0, ex - 1), np.ldexp(1.0, ex))",
        "sv[nz] = np.ldexp(1.0, ex - 1)"),
    "fp8 scale from the wrong maximum": (
        "mant, ex = np.frexp(m[nz] / FP8_E4M3_MAX)", "mant, ex = np.frexp(m[nz] / 240.0)"),
    "fp8 scores drop the row scale": (
        "out[:, v0:v1] = (h @ codes[v0:v1].astype(np.float64).T) * scales[None, v0:v1]",
        "out[:, v0:v1] = h @ codes[v0:v1].astype(np.float64).T"),
    "retrieval keeps the fp8 order": (
        "keep = np.lexsort((ids, -exact))[:K]", "keep = np.arange(K)"),
    "rescoring ties prefer the larger id": (
        "keep = np.lexsort((ids, -exact))[:K]", "keep = np.lexsort((-ids, -exact))[:K]"),
    "retrieval keeps one candidate fewer": (
        "ids = top_k(approx, R)", "ids = top_k(approx, R - 1)"),
    "conv tap before row zero": (
        "    out[1:] += (base[side, 1][None] + delta[1:, side, 1, :, None]) * Xg[:-1]\n",
        "    out += (base[side, 1][None] + delta[:, side, 1, :, None]) * np.roll(Xg, 1, axis=0)\n"),
    "conv delta rows in the wrong order": (
        "return d.reshape(X.shape[0], 2, 2, g.conv_groups)",
        "return d.reshape(X.shape[0], g.conv_groups, 2, 2).transpose(0, 2, 3, 1)"),
    "conv finish projects its own delta": (
        "o = conv_blocks(g, wts, layer, \"attn\", 1, o, d_a, W)",
        "o = conv_blocks(g, wts, layer, \"attn\", 1, o, [conv_delta(g, wts, layer, \"attn\", o[b * W:(b + 1) * W]) for b in range(B)], W)"),
    "conv sides swapped": (
        "n = conv_blocks(g, wts, layer, \"attn\", 0, n, d_a, W)",
        "n = conv_blocks(g, wts, layer, \"attn\", 1, n, d_a, W)"),
    "mlp conv prepares from the pre-norm state": (
        "d_m = [conv_delta(g, wts, layer, \"mlp\", m[b * W:(b + 1) * W]) for b in range(B)]",
        "d_m = [conv_delta(g, wts, layer, \"mlp\", y[b * W:(b + 1) * W]) for b in range(B)]"),
}


def _mutant(old, new):
    src = inspect.getsource(O)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    sys.modules["oracle_mutant"] = mod      # dataclasses look their module up here
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_tests():
    out = []
    for name, fn in inspect.getmembers(P, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            out.append((name, fn, {}))
            continue
        # expand parametrize marks (cartesian product)
        combos = [{}]
        for m in params:
            argnames = [a.strip() for a in m.args[0].split(",")]
            new = []
            for c in combos:
                for vals in m.args[1]:
                    vals = vals if len(argnames) > 1 else (vals,)
                    d = dict(c)
                    d.update(dict(zip(argnames, vals)))
                    new.append(d)
            combos = new
        for c in combos:
            out.append((name, fn, c))
    return out


@pytest.mark.parametrize("label", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(label, monkeypatch):
    old, new = MUTATIONS[label]
    mut = _mutant(old, new)
    monkeypatch.setattr(P, "O", mut)
    caught = []
    for name, fn, kw in _pin_tests():
        try:
            fn(**kw)
        except Exception:   # an assertion, or a shape/value error
            caught.append(name)
            break
    assert caught, f"no pin detects: {label}"
