"""Mutation check of the oracle's pins (CPU only).

Each mutation plants one plausible mistake in a copy of oracle/rpa_oracle.c
(a dropped term, a wrong sign or index, a swapped operand, an off-by-one
mask), builds that copy into a temporary library, and runs the pin suite
(tests/test_oracle_pins.py) against it through RPA_ORACLE_LIB. Every mutation
must make at least one pin fail: a pin suite that a broken oracle passes
would not protect the parity tests that rely on the oracle.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rpa_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text to find, replacement, which occurrence: 0-based, or None = the only one)
MUTATIONS = [
    ("gqa_value_reads_key_head", "2 * kvh + 1) * head_dim;", "2 * kvh) * head_dim;", None),
    ("gqa_key_reads_value_head", "const int64_t kbase = (row * ch + 2 * kvh) * head_dim;",
     "const int64_t kbase = (row * ch + 2 * kvh + 1) * head_dim;", None),
    ("gqa_head_map_modulo", "const int kvh = h / group;", "const int kvh = h % num_kv_heads;", None),
    ("causal_excludes_self", "if (t > p) return 0;", "if (t >= p) return 0;", None),
    ("causal_sees_next", "if (t > p) return 0;", "if (t > p + 1) return 0;", None),
    ("window_edge_off_by_one", "t <= p - window) return 0;", "t < p - window) return 0;", None),
    ("window_dropped", "if (window > 0 && t <= p - window)", "if (0 && window > 0 && t <= p - window)", None),
    ("cap_dropped", "return cap != 0.0 ? cap * tanh(s / cap) : s;", "return s;", None),
    ("cap_unscaled_tanh", "? cap * tanh(s / cap) :", "? tanh(s / cap) :", None),
    ("k_scale_dropped", "(load_elem(kv_pages, kv_dtype, kbase + d) * k_scale)",
     "load_elem(kv_pages, kv_dtype, kbase + d)", None),
    ("v_scale_dropped", "(load_elem(kv_pages, kv_dtype, vbase + d) * v_scale)",
     "load_elem(kv_pages, kv_dtype, vbase + d)", None),
    ("gqa_sm_scale_dropped", "s[n] = apply_cap(dot * sm_scale, soft_cap);",
     "s[n] = apply_cap(dot, soft_cap);", 0),
    ("mla_sm_scale_dropped", "s[n] = apply_cap(dot * sm_scale * k_scale * q_scale, soft_cap);",
     "s[n] = apply_cap(dot * k_scale * q_scale, soft_cap);", None),
    ("mla_cap_dropped", "s[n] = apply_cap(dot * sm_scale * k_scale * q_scale, soft_cap);",
     "s[n] = dot * sm_scale * k_scale * q_scale;", None),
    ("mla_q_scale_dropped", "dot * sm_scale * k_scale * q_scale", "dot * sm_scale * k_scale", None),
    ("mla_k_scale_dropped", "dot * sm_scale * k_scale * q_scale", "dot * sm_scale * q_scale", None),
    ("mla_v_scale_dropped", "o[d] = o[d] * v_scale / norm;", "o[d] = o[d] / norm;", None),
    ("gqa_q_scale_dropped", "(load_elem(q, q_dtype, qbase + d) * q_scale)",
     "load_elem(q, q_dtype, qbase + d)", None),
    ("int8_read_unsigned", "(double)((const int8_t*)base)[idx]", "(double)((const uint8_t*)base)[idx]", None),
    ("int4_nibbles_swapped", "(idx % 2 == 0) ? (b & 0xF) : (b >> 4)", "(idx % 2 == 0) ? (b >> 4) : (b & 0xF)", None),
    ("int4_unsigned", "return (double)(v < 8 ? v : v - 16);", "return (double)v;", None),
    ("int4_byte_index", "((const uint8_t*)base)[idx / 2]", "((const uint8_t*)base)[idx]", None),
    ("mla_window_dropped", "if (!key_visible(t, pos, sliding_window)) continue;",
     "if (!key_visible(t, pos, 0)) continue;", 1),
    ("gqa_no_causal_offset", "const int64_t pos = kv_len - q_len + (tok - cu_q_lens[i]);",
     "const int64_t pos = (tok - cu_q_lens[i]);", 0),
    ("mla_no_causal_offset", "const int64_t pos = kv_len - q_len + (tok - cu_q_lens[i]);",
     "const int64_t pos = (tok - cu_q_lens[i]);", 1),
    ("gqa_table_row_ignored", "page_indices[(int64_t)i * pages_per_seq + t / page_size]",
     "page_indices[t / page_size]", 0),
    ("mla_table_row_ignored", "page_indices[(int64_t)i * pages_per_seq + t / page_size]",
     "page_indices[t / page_size]", 1),
    ("gqa_row_in_page_wrong", "(int64_t)page * page_size + t % page_size; /* token row in pool */",
     "(int64_t)page * page_size + (t + 1) % page_size;", None),
    ("gqa_not_normalised", "for (int d = 0; d < head_dim; ++d) o[d] /= norm;", "", None),
    ("mla_rope_dropped", "dot += load_elem(q_pe, dtype, qr + d) *", "dot += 0.0 *", None),
    ("mla_value_column_shift", "o[d] += w[k] * load_elem(cache_kv_c, dtype, key_row[k] * kvc_stride + d);",
     "o[d] += w[k] * load_elem(cache_kv_c, dtype, key_row[k] * kvc_stride + d + 1);", None),
    ("mla_fused_rope_column_ignored", "row * kpe_stride + kpe_col + d", "row * kpe_stride + d", None),
    ("sparse_seq_len_dropped", "if (kp > qpos || kp >= kv_bound) continue;", "if (kp > qpos) continue;", None),
    ("sparse_causal_dropped", "if (kp > qpos || kp >= kv_bound) continue;", "if (kp >= kv_bound) continue;", None),
    ("sparse_ragged_request_search_left", "rid += cu_q_lens[j] <= si;", "rid += cu_q_lens[j] < si;", None),
    ("sparse_ragged_bound_not_per_request", "kv_bound = seq_lens[rid];", "kv_bound = seq_lens[0];", None),
    ("sparse_ragged_table_base_dropped", "table_base = cu_kv_lens[rid] / page_size;", "table_base = 0;", None),
    ("sparse_ragged_no_clip", "if (rid > num_seqs - 1) rid = num_seqs - 1;", "if (rid > num_seqs) rid = num_seqs;", None),
    ("sparse_padding_as_unit0", "if (u < 0) continue;", "if (u < -1) continue;", None),
    ("sparse_row_mod_read_block", "(int64_t)page * page_size + kp % page_size;",
     "(int64_t)page * page_size + kp % read_block;", None),
    ("update_pad_not_zeroed", "memset(db, 0, (size_t)stride_b * eb);", "", None),
    ("update_k_to_value_head", "(slot * 2 * heads + 2 * h) * row_a,",
     "(slot * 2 * heads + 2 * h + 1) * row_a,", None),
    ("update_int4_row_bytes", "dtype == OR_INT4 ? dim_a / 2 :", "dtype == OR_INT4 ? dim_a :", None),
    ("update_position_off_by_one", "const int64_t pos = kv_lens[i] - q_len + (t - cu_q_lens[i]);",
     "const int64_t pos = kv_lens[i] - q_len + (t - cu_q_lens[i]) - 1;", None),
    ("e4m3_exponent_bias", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)", None),
    ("e4m3_subnormal_scale", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)", None),
]


def _mutate(text, find, repl, occ):
    n = text.count(find)
    if occ is None:
        assert n == 1, f"{find!r} occurs {n} times"
        return text.replace(find, repl)
    assert n > occ, f"{find!r} occurs {n} times, occurrence {occ} asked"
    start = -1
    for _ in range(occ + 1):
        start = text.index(find, start + 1)
    return text[:start] + repl + text[start + len(find):]


def _run_one(m, tmp):
    name, find, repl, occ = m
    with open(SRC) as f:
        text = _mutate(f.read(), find, repl, occ)
    src = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib,
                           src, "-lm"], stderr=subprocess.DEVNULL)
    env = dict(os.environ, RPA_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        workers = max(1, min(8, (os.cpu_count() or 2)))
        with cf.ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(lambda m: _run_one(m, tmp), MUTATIONS))
        # A run that ended oddly (neither a pass nor a failed pin: a crash, a
        # collection error) is run once more on its own before it counts, so
        # a one-off hiccup of the parallel runs does not read as a finding.
        by_name = {m[0]: m for m in MUTATIONS}
        results = [(name, rc if rc in (0, 1) else _run_one(by_name[name], tmp)[1])
                   for name, rc in results]
    survived = [name for name, rc in results if rc == 0]
    assert not survived, f"mutations no pin catches: {survived}"
    # rc 1 = a test failed; anything else (collection error, crash) is not a pin catching it.
    odd = [(name, rc) for name, rc in results if rc not in (0, 1)]
    assert not odd, f"mutations that broke the run instead of failing a pin: {odd}"


@pytest.mark.parametrize("m", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_applies(m):
    with open(SRC) as f:
        text = f.read()
    assert _mutate(text, m[1], m[2], m[3]) != text
