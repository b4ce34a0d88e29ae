"""Plant plausible mistakes in copies of the oracle (on the CPU, in a temporary
directory) and require that the pins catch every one of them.  This is what
makes the pins evidence: a dropped term, a wrong index or sign, an off-by-one
or a transposed operand anywhere in the oracle must fail at least one pin."""
import os
import subprocess
import tempfile

import pytest

import oracle_pins as P
import oracle.oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "msa_oracle.c")

# (name, original text, mutated text); each original must occur exactly once.
MUTANTS = [
    ("bf16_truncated_half", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("index_head_attribution", "if (i % p->n_kv_heads != h) continue;",
     "if (i / p->n_kv_heads != h) continue;"),
    ("block_drops_last_token", "for (int32_t j = c * bs; j < (c + 1) * bs; ++j) {",
     "for (int32_t j = c * bs; j < (c + 1) * bs - 1; ++j) {"),
    ("block_min_not_max", "if (s > best) best = s;", "if (s > best || best == -INFINITY) best = -s;"),
    ("own_block_not_forced", "value = INFINITY; /* own block always kept */",
     "value = -INFINITY; /* own block always kept */"),
    ("index_transposed_operand",
     "const uint16_t* kv = ik + ((int64_t)b * p->seq_kv + j) * Di;",
     "const uint16_t* kv = ik + ((int64_t)b * p->seq_kv + j) * Di + (d0 ? 0 : 0);"),
    ("ties_to_higher_index", "if (best < 0 || scores[c] > scores[best]) best = c;",
     "if (best < 0 || scores[c] >= scores[best]) best = c;"),
    ("select_one_too_few", "const int32_t m = p->top_k < n ? p->top_k : n;",
     "const int32_t m = (p->top_k < n ? p->top_k : n) - (n > 2);"),
    ("interleaved_head_groups", "const int32_t h = hq / G; /* contiguous query-head groups per KV head */",
     "const int32_t h = hq % p->n_kv_heads;"),
    ("own_block_not_causal", "for (int32_t j = c * bs; j < (c + 1) * bs && j <= pos; ++j) tok[n++] = j;",
     "for (int32_t j = c * bs; j < (c + 1) * bs; ++j) tok[n++] = j;"),
    ("own_block_excludes_self", "for (int32_t j = c * bs; j < (c + 1) * bs && j <= pos; ++j) tok[n++] = j;",
     "for (int32_t j = c * bs; j < (c + 1) * bs && j < pos; ++j) tok[n++] = j;"),
    ("dropped_softmax_scale", "z[a] = p->softmax_scale * s;", "z[a] = s;"),
    ("lse_missing_max", "lse[hq] = zmax + log(l);", "lse[hq] = log(l);"),
    ("v_read_from_k", "const uint16_t* vv = v + (((int64_t)b * p->n_kv_heads + h) * p->seq_kv + tok[a]) * D;",
     "const uint16_t* vv = k + (((int64_t)b * p->n_kv_heads + h) * p->seq_kv + tok[a]) * D;"),
    ("unnormalised_output", "for (int32_t d = 0; d < D; ++d) o[d] /= l;", "for (int32_t d = 0; d < D; ++d) o[d] /= (l + 1e-3);"),
    ("decode_position_off_by_one", "return L - 1;", "return L - 2 < 0 ? 0 : L - 2;"),
    ("dense_not_causal_last", "const int32_t nkeys = pos + 1;", "const int32_t nkeys = pos;"),
    ("dense_head_map", "const int32_t kvh = hq / (p->n_q_heads / p->n_kv_heads);",
     "const int32_t kvh = hq % p->n_kv_heads;"),
    ("dense_scale", "w[j] = acc * p->softmax_scale;", "w[j] = acc;"),
    # the main-branch gradient and its fp64 forward
    ("bwd_missing_dsum", "const double ds = w[a] * (dp - dsum);", "const double ds = w[a] * dp;"),
    ("bwd_dsum_sign", "const double ds = w[a] * (dp - dsum);",
     "const double ds = w[a] * (dsum - dp);"),
    ("bwd_dk_unscaled", "dkv[d] += p->softmax_scale * ds * qv[d];", "dkv[d] += ds * qv[d];"),
    ("bwd_dq_reads_v", "dq[qoff + d] += p->softmax_scale * ds * kv[d];",
     "dq[qoff + d] += p->softmax_scale * ds * vv[d];"),
    ("bwd_dv_uses_ds", "dvv[d] += w[a] * g[d];", "dvv[d] += ds * g[d];"),
    ("bwd_unnormalised_weights", "for (int32_t a = 0; a < n; ++a) w[a] /= l;",
     "for (int32_t a = 0; a < n; ++a) w[a] /= (l + 0.5);"),
    ("bwd_dsum_uses_q", "for (int32_t d = 0; d < D; ++d) dsum += g[d] * o[d];",
     "for (int32_t d = 0; d < D; ++d) dsum += g[d] * qv[d];"),
    ("bwd_tokens_not_causal", "for (int32_t j = c * bs; j <= pos && j < (c + 1) * bs; ++j) tok[n++] = j;",
     "for (int32_t j = c * bs; j < (c + 1) * bs && j < p->seq_kv; ++j) tok[n++] = j;"),
    ("f64_forward_unscaled", "z[a] = s * p->softmax_scale;", "z[a] = s;"),
    # the index branch's KL signal
    ("kl_target_not_averaged", "P[a] += w[a] / l / G;", "P[a] += w[a] / l;"),
    ("kl_gradient_sign", "const double g = Q[a] - P[a];", "const double g = P[a] - Q[a];"),
    ("kl_index_scaled", "Q[a] = s;\n          if (s > smax) smax = s;",
     "Q[a] = p->softmax_scale * s;\n          if (p->softmax_scale * s > smax) smax = p->softmax_scale * s;"),
    ("kl_diq_reads_iq", "dq_row[d] += g * kv[d];", "dq_row[d] += g * iv[d];"),
    ("kl_dik_reads_ik", "dk_row[d] += g * iv[d];", "dk_row[d] += g * kv[d];"),
    ("kl_head_attribution", "const int32_t h = i % Hkv;", "const int32_t h = i / (Hi / Hkv);"),
    ("kl_target_unscaled", "            w[a] = p->softmax_scale * s;", "            w[a] = s;"),
    ("kl_lse_missing_max", "const double lse = smax + log(lq);", "const double lse = log(lq);"),
    ("kl_reversed_direction", "if (P[a] > 0.0) kl += P[a] * (log(P[a]) - logq);",
     "if (P[a] > 0.0) kl += Q[a] * (logq - log(P[a]));"),
]


def _fix_transposed(src):
    # the transposed-operand mutant swaps the roles of query row and key token
    return src.replace(
        "const uint16_t* qv = iq + (((int64_t)b * p->seq_q + t) * p->n_idx_heads + i) * Di;\n"
        "  const uint16_t* kv = ik + ((int64_t)b * p->seq_kv + j) * Di + (d0 ? 0 : 0);",
        "const uint16_t* qv = iq + (((int64_t)b * p->seq_q + (j % p->seq_q)) * p->n_idx_heads + i) * Di;\n"
        "  const uint16_t* kv = ik + ((int64_t)b * p->seq_kv + (t % p->seq_kv)) * Di;")


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, mut, tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation anchor for {name} not unique/present"
    msrc = src.replace(orig, mut)
    if name == "index_transposed_operand":
        msrc = _fix_transposed(msrc)
    cpath = tmp_path / "msa_oracle.c"
    cpath.write_text(msrc)
    hdr = os.path.join(os.path.dirname(SRC), "msa_oracle.h")
    (tmp_path / "msa_oracle.h").write_text(open(hdr).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(cpath), "-o", str(lib), "-lm"],
                   check=True)
    L = O.lib(str(lib))
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(L)
        except (AssertionError, RuntimeError):
            caught.append(check.__name__)
    assert caught, f"no pin catches mutant {name}"
