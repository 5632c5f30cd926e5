"""Planted mistakes in copies of the oracle's C source must each fail at least one pin.

This shows that the pins constrain every part of the oracle: the block-table
dereference, the head mapping, the causal horizon, the softmax, the scale, the
normalisation, the operand choice, the bf16 widening, and the KV-cache write's
position, slot, source row and element copy, and the block copy's
ids, slots, heads and pairs. Mutants are compiled
with gcc into a temporary directory on the CPU; the real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

from oracle.oracle import _SRC, build

RUNNER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_run_pins.py")


def _run_pins(lib):
    """Run the pin battery in a child process; a crash or a hang (a mutant that writes out of bounds can
    corrupt the heap) counts as caught."""
    env = dict(os.environ, OMP_NUM_THREADS="2")
    try:
        r = subprocess.run([sys.executable, RUNNER, lib], capture_output=True, text=True, timeout=120, env=env)
    except subprocess.TimeoutExpired:
        return -1, ["FAIL timeout"], []
    lines = r.stdout.splitlines()
    return r.returncode, [ln for ln in lines if ln.startswith("FAIL")], [ln for ln in lines if ln.startswith("PASS")]

MUTANTS = {
    "block index uses slot": ("i / p->block_size]", "i % p->block_size]"),
    "slot uses block index": ("int slot = i % p->block_size;", "int slot = i / p->block_size;"),
    "gqa head mapping modulo": ("const int g = h / group;", "const int g = h % p->num_kv_heads;"),
    "causal horizon off by one": ("return ctx - q_len + j + 1;", "return ctx - q_len + j;"),
    "causal mask top-left aligned": ("return ctx - q_len + j + 1;", "return j + 1;"),
    "no max subtraction": ("x[i] = exp(x[i] - m);", "x[i] = exp(x[i]);"),
    "minimum instead of maximum": ("if (x[i] > m) m = x[i];", "if (x[i] < m) m = x[i];"),
    "normalise by count": ("out[d] /= z;", "out[d] /= n;"),
    "weights summed as ones": ("z += x[i];", "z += 1.0;"),
    "scale dropped": ("x[i] = p->scale * dot;", "x[i] = dot;"),
    "kv stride uses query heads": ("* p->num_kv_heads + g) * p->head_dim;", "* p->num_q_heads + g) * p->head_dim;"),
    "keys used as values": ("element(p, p->v_cache, v_off + d)", "element(p, p->k_cache, v_off + d)"),
    "key element index dropped": ("element(p, p->k_cache, k_off + d)", "element(p, p->k_cache, k_off)"),
    "query row of request not token": ("((int64_t)t * p->num_q_heads + h) * D;", "((int64_t)s * p->num_q_heads + h) * D;"),
    "bf16 widening shift": ("<< 16;", "<< 15;"),
    "last visible key skipped": ("for (int i = 0; i < n; ++i) {\n    int64_t k_off", "for (int i = 0; i < n - 1; ++i) {\n    int64_t k_off"),
    "value loop skips last key": ("for (int i = 0; i < n; ++i) {\n    int64_t v_off", "for (int i = 0; i < n - 1; ++i) {\n    int64_t v_off"),
    # KV-cache write
    "cache write position off by one": ("const int pos = ctx - q_len + j;", "const int pos = ctx - q_len + j + 1;"),
    "cache write slot uses block index": ("const int slot = pos % block_size;", "const int slot = pos / block_size;"),
    "cache write row of request not token": ("const size_t src = ((size_t)t * row_elems", "const size_t src = ((size_t)s * row_elems"),
    "cache write values from keys": ("((const unsigned char*)v_new)[src + b]", "((const unsigned char*)k_new)[src + b]"),
    "cache write first element only": ("for (size_t e = 0; e < row_elems; ++e) {", "for (size_t e = 0; e < 1; ++e) {"),
    "cache write position from start": ("const int pos = ctx - q_len + j;", "const int pos = j;"),
    # block copy
    "copy values from keys": ("((const unsigned char*)src_v)[src + b]", "((const unsigned char*)src_k)[src + b]"),
    "copy source addressed by destination id": ("((size_t)from * block_size + slot)", "((size_t)to * block_size + slot)"),
    "copy mapping columns swapped": ("const int32_t from = mapping[2 * i], to = mapping[2 * i + 1];\n    for (int slot",
                                     "const int32_t to = mapping[2 * i], from = mapping[2 * i + 1];\n    for (int slot"),
    "copy skips last slot": ("for (int slot = 0; slot < block_size; ++slot)", "for (int slot = 0; slot < block_size - 1; ++slot)"),
    "copy first kv head only": ("for (int g = 0; g < num_kv_heads; ++g)", "for (int g = 0; g < 1; ++g)"),
    "copy first pair only": ("i < num_pairs; ++i) {\n    const int32_t from = mapping[2 * i], to = mapping[2 * i + 1];\n    for",
                             "i < 1; ++i) {\n    const int32_t from = mapping[2 * i], to = mapping[2 * i + 1];\n    for"),
    "copy accepts ids past the pool": ("from >= src_num_blocks ||", "from > src_num_blocks ||"),
}


@pytest.fixture(scope="module")
def source():
    with open(_SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = build(str(src), str(tmp_path / "libmutant.so"))
    rc, failed, _ = _run_pins(lib)
    assert rc != 0 or failed, f"no pin caught the planted mistake '{name}'"


def test_unmutated_copy_passes(source, tmp_path):
    src = tmp_path / "same.c"
    src.write_text(source)
    lib = build(str(src), str(tmp_path / "libsame.so"))
    rc, failed, passed = _run_pins(lib)
    assert rc == 0 and not failed and passed
