"""The oracle's pins are sensitive: plant a plausible mistake in a copy of the
oracle (on the CPU, in a temporary directory) and check that a pin fails."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    # (file, original, planted mistake, pin test that must fail)
    ("oracle/accept.py", "w = np.maximum(0.0, p - q)", "w = np.maximum(0.0, q - p)",
     "test_oracle_accept.py::test_first_token_law_is_p_by_integration_over_uniforms"),
    ("oracle/accept.py", "y, m = _inverse_cdf(w, float(u_all[t0 + D]))",
     "y, m = _inverse_cdf(w, float(u_all[t0 + n]))",
     "test_oracle_accept.py::test_tiny_workload_emitted_tokens_follow_p_chi_square"),
    ("oracle/accept.py", "r = float(np.exp(np.float64(lp - lq)))", "r = float(np.exp(np.float64(lq - lp)))",
     "test_oracle_accept.py::test_first_token_law_is_p_by_integration_over_uniforms"),
    ("oracle/accept.py", "        out[t0 + n] = int(np.argmax(target[t0 + n]))",
     "        out[t0 + n] = int(np.argmax(target[t0 + max(n - 1, 0)]))",
     "test_oracle_accept.py::test_greedy_speculation_equals_plain_greedy_decoding"),
    ("oracle/accept.py", 'j = int(np.searchsorted(C, T, side="right"))', 'j = int(np.searchsorted(C[::-1], T))',
     "test_oracle_accept.py::test_d0_is_inverse_cdf_sampling_of_p"),
    ("oracle/attention.py", "P = n - rows + i", "P = n - rows + i - 1",
     "test_oracle_attention.py::test_matches_sdpa_lower_right_causal"),
    ("oracle/attention.py", "Qg = bf16_bits_to_f64(q_bits[t0 + i, h * group:(h + 1) * group, :])",
     "Qg = bf16_bits_to_f64(q_bits[t0 + i, h::k_bits.shape[1]][:group])",
     "test_oracle_attention.py::test_matches_sdpa_lower_right_causal"),
    ("oracle/attention.py", "return bf16_bits_to_f64(cache_bits[pages, h, j % ps, :])",
     "return bf16_bits_to_f64(cache_bits[pages, h, (j // ps) % ps, :])",
     "test_oracle_attention.py::test_matches_sdpa_lower_right_causal"),
    # draft trees
    ("oracle/tree.py", "anc.append(anc[p] | {i})", "anc.append({0, i})",
     "test_oracle_tree.py::test_chain_tree_is_the_causal_block"),
    ("oracle/tree.py", "accepted[i] = accepted[p] and 0 <= x < V and x == top[p]",
     "accepted[i] = accepted[p] and 0 <= x < V and x == top[i]",
     "test_oracle_tree.py::test_chain_acceptance_is_linear_greedy"),
    ("oracle/tree.py", "if accepted[i] and depth[i] > depth[best]:", "if accepted[i] and depth[i] >= depth[best]:",
     "test_oracle_tree.py::test_acceptance_matches_path_enumeration"),
    # relaxed acceptance
    ("oracle/lossy.py", "return math.sqrt(max(0.0, 0.5 * (kp + kq)))", "return max(0.0, 0.5 * (kp + kq))",
     "test_oracle_lossy.py::test_statistics_match_scipy"),
    ("oracle/lossy.py", "                if not strict:", "                if strict:",
     "test_oracle_lossy.py::test_negative_threshold_is_the_lossless_rule"),
    ("oracle/lossy.py", "ent[d0 + i] = row_entropy(draft[d0 + i])", "ent[d0 + i] = row_entropy(target[t0 + i])",
     "test_oracle_lossy.py::test_negative_threshold_is_the_lossless_rule"),
    # closed loop
    ("oracle/loop.py", "for j in range(L - k - 1, -1, -1):", "for j in range(0, L - k):",
     "test_oracle_loop.py::test_ngram_drafter_by_hand"),
    ("oracle/loop.py", "        if d >= ema:", "        if d > ema:", "test_oracle_loop.py::test_tier_rule_by_hand"),
    ("oracle/loop.py", "            rows.append(h[-1])", "            rows.append(h[-2] if len(h) > 1 else h[-1])",
     "test_oracle_loop.py::test_loop_output_is_plain_greedy_decoding"),
    # verify-shaped linear layer
    ("oracle/gemm.py", "if a.dtype in (np.uint16, np.int16):", "if a.dtype in (np.int16,):",
     "test_oracle_gemm.py::test_identity_weight_returns_x"),
    ("oracle/gemm.py", "return np.abs(_widen(x)) @ np.abs(_widen(w)).T", "return np.abs(_widen(x) @ _widen(w).T)",
     "test_oracle_gemm.py::test_abs_sum_brute_force"),
    ("oracle/gemm.py", "return np.abs(_widen(x)) @ np.abs(_widen(w)).T", "return 2.0 * np.abs(_widen(x)) @ np.abs(_widen(w)).T",
     "test_oracle_gemm.py::test_abs_sum_brute_force"),
]


@pytest.mark.parametrize("path,old,new,pin", MUTATIONS, ids=[f"m{i}" for i in range(len(MUTATIONS))])
def test_planted_mistake_fails_a_pin(tmp_path, path, old, new, pin):
    for d in ("oracle", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "golden"))
    src = (tmp_path / path).read_text()
    assert old in src, "mutation anchor drifted from the oracle source"
    (tmp_path / path).write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        f"tests/{pin}"], cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, r.stdout[-2000:]
    assert "failed" in r.stdout
