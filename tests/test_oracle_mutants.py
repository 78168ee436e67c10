"""Each planted mistake in a copy of the oracle must make at least one pin fail.

The mistakes are the plausible ones: a wrong index or feature order, a dropped
term, a wrong sign, a transposed operand, a wrong padding rule, a missing check.
"""
import os

import pytest

import pins
from oracle import oracle as o

SRC = open(os.path.join(os.path.dirname(o.__file__), "vlb_oracle.c")).read()

MUTANTS = {
    "feature order dx/dy swapped": (
        "out[t * K1 + (int64_t)c * k * k + dy * k + dx] =",
        "out[t * K1 + (int64_t)c * k * k + dx * k + dy] ="),
    "position-major features in the row path": (
        "out[(int64_t)c * k * k + dy * k + dx] = inside",
        "out[(int64_t)(dy * k + dx) * C + c] = inside"),
    "merged side rounds down": ("while (g_pad % k != 0) g_pad++;", "g_pad -= g_pad % k;"),
    "padding at the low end": ("if (y >= gh || xx >= gw) return 0.0;\n  return x[(y * gw + xx) * C + c];",
                               "int64_t oy = y - (k_pad_h), ox = xx;\n  (void)ox; if (oy < 0 || y >= gh + 0 || xx >= gw) return 0.0;\n  return x[(oy * gw + xx) * C + c];"),
    "unbiased variance": ("var /= C;\n    double inv", "var /= (C - 1);\n    double inv"),
    "eps outside the square root": ("double inv = 1.0 / sqrt(var + eps)",
                                    "double inv = 1.0 / (sqrt(var) + eps)"),
    "gamma and beta swapped": ("* inv * gamma[c] + beta[c]", "* inv * beta[c] + gamma[c]"),
    "bias dropped": ("j->out[r * j->out_dim + o] = acc + (j->b ? j->b[o] : 0.0);",
                     "j->out[r * j->out_dim + o] = acc;"),
    "weight transposed": ("acc += a[i] * w[i];",
                          "acc += a[i] * j->W[(int64_t)i * j->out_dim + o]; (void)w;"),
    "gelu sign": ("(1.0 + erf(x[i] / sqrt(2.0)))", "(1.0 - erf(x[i] / sqrt(2.0)))"),
    "gelu scale": ("erf(x[i] / sqrt(2.0))", "erf(x[i] / 2.0)"),
    "no local transpose": ("base + (1 + i * tw + j) * per_view + y * wp + x",
                           "base + (1 + i * tw + j) * per_view + x * wp + y"),
    "newline per local view": ("          n = emit(src, cap, n, base + (1 + i * tw + j) * per_view + y * wp + x);\n      n = emit(src, cap, n, ORC_SRC_NEWLINE);",
                               "          n = emit(src, cap, n, base + (1 + i * tw + j) * per_view + y * wp + x);\n      n = emit(src, cap, n, ORC_SRC_NEWLINE); if (tw > 1) n = emit(src, cap, n, ORC_SRC_NEWLINE);"),
    "separator before the global view": (
        "      n = emit_global(src, cap, n, row, hp, wp);\n      n = emit(src, cap, n, ORC_SRC_SEPARATOR);",
        "      n = emit(src, cap, n, ORC_SRC_SEPARATOR);\n      n = emit_global(src, cap, n, row, hp, wp);"),
    "placeholder formula without local newlines": ("(th * hp) * (tw * wp + 1)", "(th * hp) * (tw * wp)"),
    "scatter in reverse": ("    if (!mask[i]) continue;\n    const double *from = src[j] >= 0                  ? rows + src[j] * D",
                           "    if (!mask[i]) continue;\n    j = P - 1 - j; const double *from = src[j] >= 0 ? rows + src[j] * D"),
    # count-check mutants keep rejecting too many placeholders: with more
    # placeholders than slots the mutated code would read past the slot list
    "count check misses too few placeholders": ("if (count != P) return -1;\n  int64_t j = 0;",
                                                "if (count > P) return -1;\n  int64_t j = 0;"),
    "param count without second bias": ("hidden * out_dim + out_dim;", "hidden * out_dim;"),
    "embedding row off by one": ("const int64_t e = (int64_t)ids[i] * D;",
                                 "const int64_t e = (int64_t)(ids[i] > 0 ? ids[i] - 1 : 0) * D;"),
    "embedding keeps text positions at zero": (
        "for (int32_t d = 0; d < D; d++) to[d] = e_bf16 ? bf16_bits(e_bf16[e + d]) : e_f64[e + d];",
        "for (int32_t d = 0; d < D; d++) to[d] = 0.0 * e;"),
    "embedding without the id range check": ("if (bad_id) return -2;", "(void)bad_id;"),
    "embedding count check misses too few": ("if (n_img != P) return -1;",
                                             "if (n_img > P) return -1;"),
    "embedding places visual rows in reverse": (
        "      const double *from = src[j] >= 0                  ? rows + src[j] * D\n                           : src[j] == ORC_SRC_NEWLINE ? newline",
        "      const int64_t jj = P - 1 - j;\n      const double *from = src[jj] >= 0                 ? rows + src[jj] * D\n                           : src[jj] == ORC_SRC_NEWLINE ? newline"),
    "bf16 table widened as the low half": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h;"),
    "middle Linear without its activation": ("    for (int32_t q = 0; q < s->n_mid; q++) {\n      apply_act(s->act, h, H);",
                                             "    for (int32_t q = 0; q < s->n_mid; q++) {\n      (void)0;"),
    "middle Linears in reverse order": ("orc_linear(h, 1, H, j->W_mid + (int64_t)q * H * H, j->b_mid + (int64_t)q * H, H, h2, 1);",
                                        "orc_linear(h, 1, H, j->W_mid + (int64_t)(s->n_mid - 1 - q) * H * H, j->b_mid + (int64_t)(s->n_mid - 1 - q) * H, H, h2, 1);"),
    # backward
    "gelu slope without the z*phi term": (
        "return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * exp(-0.5 * z * z) / sqrt(2.0 * M_PI);",
        "return 0.5 * (1.0 + erf(z / sqrt(2.0)));"),
    "tanh slope without the inner derivative": (
        "* a * (1.0 + 3.0 * 0.044715 * z * z);", "* a;"),
    "dW2 from the pre-activation": ("dW2[(int64_t)o * H + h] += dy[o] * act_value(s->act, z[h]);",
                                    "dW2[(int64_t)o * H + h] += dy[o] * z[h];"),
    "dW2 transposed": ("dW2[(int64_t)o * H + h] += dy[o] * act_value(s->act, z[h]);",
                       "dW2[(int64_t)h * O + o] += dy[o] * act_value(s->act, z[h]);"),
    "db2 dropped": ("for (int32_t o = 0; o < O; o++) db2[o] += dy[o];",
                    "for (int32_t o = 0; o < O; o++) db2[o] += 0.0 * dy[o];"),
    "activation gradient without the slope": ("dz[h] = da * act_slope(s->act, z[h]);",
                                              "dz[h] = da;"),
    "dA through W2 transposed": (
        "        for (int32_t o = 0; o < O; o++) da += dy[o] * W2[(int64_t)o * H + h];\n        dz[h]",
        "        for (int32_t o = 0; o < O; o++) da += dy[o] * W2[(int64_t)h * O + o];\n        dz[h]"),
    "dW1 row and column swapped": ("for (int64_t i = 0; i < K1; i++) dW1[h * K1 + i] += dz[h] * m[i];",
                                   "for (int64_t i = 0; i < K1; i++) dW1[i * H + h] += dz[h] * m[i];"),
    "db1 before the slope": ("db1[h] += dz[h];", "db1[h] += dz[h] / act_slope(s->act, z[h]);"),
    "dm through W1 with the wrong stride": ("for (int32_t h = 0; h < H; h++) acc += dz[h] * W1[h * K1 + i];",
                                            "for (int32_t h = 0; h < H; h++) acc += dz[h] * W1[h * K1 + (i + 1) % K1];"),
    "unmerge dx/dy swapped": ("= dm[(int64_t)c * k * k + ddy * k + ddx];",
                              "= dm[(int64_t)c * k * k + ddx * k + ddy];"),
    "LN backward without mean(g)": ("dx[c] = r * (gamma[c] * dn[c] - mg - xh * mgx);",
                                    "dx[c] = r * (gamma[c] * dn[c] - xh * mgx);"),
    "LN backward without the xh term": ("dx[c] = r * (gamma[c] * dn[c] - mg - xh * mgx);",
                                        "dx[c] = r * (gamma[c] * dn[c] - mg);"),
    "LN backward ignores gamma": ("const double xh = (x[c] - mean) * r, g = gamma[c] * dn[c];",
                                  "const double xh = (x[c] - mean) * r, g = dn[c];"),
    "LN backward eps outside the root": ("const double r = 1.0 / sqrt(var + eps);",
                                         "const double r = 1.0 / (sqrt(var) + eps);"),
    "dgamma and dbeta swapped": ("if (dgamma) dgamma[c] += dn[c] * xh;\n    if (dbeta) dbeta[c] += dn[c];",
                                 "if (dgamma) dgamma[c] += dn[c];\n    if (dbeta) dbeta[c] += dn[c] * xh;"),
    "scatter backward keeps the last newline only": ("for (int32_t d = 0; d < D; d++) to[d] += g[d];",
                                                     "for (int32_t d = 0; d < D; d++) to[d] = g[d];"),
    "scatter backward count check misses too few": ("if (count != P) return -1;\n  memset(drows",
                                                    "if (count > P) return -1;\n  memset(drows"),
    "middle dW from the pre-activation": ("dW_mid[((int64_t)q * H + j) * H + h] += dz[j] * act_value(s->act, zq[h]);",
                                          "dW_mid[((int64_t)q * H + j) * H + h] += dz[j] * zq[h];"),
    "middle backward without the slope": ("dzp[h] = da * act_slope(s->act, zq[h]);", "dzp[h] = da;"),
    "middle dA through W transposed": ("da += dz[j] * Wq[(int64_t)j * H + h];",
                                       "da += dz[j] * Wq[(int64_t)h * H + j];"),
    "middle bias gradient dropped": ("db_mid[(int64_t)q * H + j] += dz[j];",
                                     "db_mid[(int64_t)q * H + j] += 0.0 * dz[j];"),
    "sampled unit misses the bias": ("    z += b1[h];\n    const double a = act_value(s->act, z);",
                                     "    const double a = act_value(s->act, z);"),
    "sampled pixel at the transposed block position": ("const int32_t p = (y % k) * k + xx % k;",
                                                       "const int32_t p = (xx % k) * k + y % k;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not unique/found: {name}"
    text = SRC.replace(old, new)
    if "k_pad_h" in new:
        text = text.replace("static double padded_cell(", "static int k_pad_h = 1;\nstatic double padded_cell(")
    so = o.build_variant(text, str(tmp_path), "mut")
    with o.use_library(so):
        bad = pins.failing(o)
    assert bad, f"no pin catches: {name}"


# ---- the processor oracle (pure Python): planted mistakes, caught by its pins ----
PR_SRC = open(os.path.join(os.path.dirname(o.__file__), "processor.py")).read()

PR_MUTANTS = {
    "scale as max": ("        scale = min(W / w0, H / h0)\n", "        scale = max(W / w0, H / h0)\n"),
    "effective not capped": ("eff = min(math.floor(w0 * scale) * math.floor(h0 * scale), w0 * h0)",
                             "eff = math.floor(w0 * scale) * math.floor(h0 * scale)"),
    "floor of the product": ("eff = min(math.floor(w0 * scale) * math.floor(h0 * scale), w0 * h0)",
                             "eff = min(math.floor(w0 * scale * h0 * scale), w0 * h0)"),
    "waste tie-break reversed": ("(eff == best_eff and waste < best_waste)",
                                 "(eff == best_eff and waste > best_waste)"),
    "last of full ties": ("(eff == best_eff and waste < best_waste)",
                          "(eff == best_eff and waste <= best_waste)"),
    "crop for three images": ("MAX_CROP_IMAGES = 2", "MAX_CROP_IMAGES = 3"),
    "tiles height first": ("tw, th = best[0] // image_size, best[1] // image_size",
                           "th, tw = best[0] // image_size, best[1] // image_size"),
    "merged side rounds down": ("return -(-(image_size // patch_size) // downsample)",
                                "return (image_size // patch_size) // downsample"),
    "no BOS": ("out, i = [bos_id], 0", "out, i = [], 0"),
    "one image token per image": ("out.extend([image_token_id] * slots[i])",
                                  "out.extend([image_token_id] * 1)"),
    "counts in reverse": ("out.extend([image_token_id] * slots[i])",
                          "out.extend([image_token_id] * slots[len(slots) - 1 - i])"),
    "no prompt check": ("    if sum(1 for t in ids if t == image_token_id) != len(slots):\n        raise ValueError",
                        "    if False:\n        raise ValueError"),
}


@pytest.mark.parametrize("name", sorted(PR_MUTANTS))
def test_processor_mutant_is_caught(name):
    import types
    old, new = PR_MUTANTS[name]
    assert PR_SRC.count(old) == 1, f"mutation anchor not unique/found: {name}"
    mod = types.ModuleType("processor_mutant")
    exec(compile(PR_SRC.replace(old, new), "processor_mutant", "exec"), mod.__dict__)
    bad = []
    for p in pins.PROCESSOR_PINS:
        try:
            p(o, mod)
        except Exception:  # noqa: BLE001 - any failure counts
            bad.append(p.__name__)
    assert bad, f"no pin catches: {name}"
