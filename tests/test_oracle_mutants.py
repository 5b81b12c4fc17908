"""The oracle's pins are not vacuous: each test here plants one plausible
mistake in a copy of the oracle's C source (a swapped nibble order, a wrong
constant, a dropped term, a wrong index...), builds it on the CPU, and
checks that the pins covering that function fail against it."""
import os
import subprocess

import pytest

import oracle
import test_context_chunks_cpu as chunks
import test_kv_views_cpu as views
import test_oracle_ops as ops
import test_sparse_index_cpu as sparse
from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "gcache_oracle.c")

# A binary32 value rounded to odd from an exact double: rounding it to bf16
# afterwards equals one correct rounding of the exact value (binary32 keeps
# more than two extra bits), so a mutant built with it rounds only once.
ROUND_ONCE = ("({ double d_ = (%s); float f_ = (float)d_; "
              "if (fabs((double)f_) > fabs(d_)) f_ = nextafterf(f_, 0.0f); "
              "if ((double)f_ != d_) { uint32_t u_; memcpy(&u_, &f_, 4); u_ |= 1u; memcpy(&f_, &u_, 4); } f_; })")

# (name, text in the oracle source, replacement, pins that must catch it)
MUTANTS = [
    ("nibble order", "entry[k] = (uint8_t)(q[2 * k] | (q[2 * k + 1] << 4));",
     "entry[k] = (uint8_t)(q[2 * k + 1] | (q[2 * k] << 4));",
     [ops.test_nvfp4_block_hand_vectors, ops.test_nvfp4_write_and_gathers_vs_brute_force_tiny]),
    ("scale divisor", "uint8_t sf = orc_e4m3_encode(amax / 6.0f);", "uint8_t sf = orc_e4m3_encode(amax / 4.0f);",
     [ops.test_nvfp4_block_hand_vectors, ops.test_page_tolerances_tiny_and_decode_workloads]),
    ("walk drops the request start", "+ (r - ws[req]);", "+ r;",
     [ops.test_gather_walk_hand_vectors, ops.test_address_tags_pin_the_walk]),
    ("fp8 group index", "* sc[i / F8_GROUP];", "* sc[0];",
     [ops.test_fp8_hand_vectors, ops.test_fp8_write_and_gather_vs_brute_force]),
    ("per-head scale without gs", "float e = orc_e4m3_decode(sf) * gs;", "float e = orc_e4m3_decode(sf);",
     [ops.test_perhead_hand_vectors]),
    ("bf16 byte order", "row[i] = (uint16_t)(entry[2 * i] | (entry[2 * i + 1] << 8));",
     "row[i] = (uint16_t)(entry[2 * i + 1] | (entry[2 * i] << 8));",
     [ops.test_bf16_comparator_gather_vs_brute_force]),
    ("chunk membership", "if (p / chunk_rows == chunk) rows++;", "if (p / chunk_rows <= chunk) rows++;",
     [chunks.test_oracle_chunk_plan_hand_vectors, chunks.test_oracle_chunk_plan_invariants]),
    ("slot offset", "result = blk * block_size + i % block_size;", "result = blk * block_size + i / block_size;",
     [sparse.test_hand_vectors, sparse.test_random_vs_brute_force]),
    ("HND token stride", "out->data_token_stride = data_row;", "out->data_token_stride = data_per_head;",
     [views.test_split_layout_hand_values]),
    # rounding-order readings: only the hand vectors are listed, the brute
    # force restates the same formulas
    ("fp8 write divides by the scale", "entry[i] = orc_e4m3_encode(orc_bf16_to_f32(nope[i]) * inv);",
     "entry[i] = orc_e4m3_encode(orc_bf16_to_f32(nope[i]) / sc);",
     [ops.test_fp8_rounding_order_hand_vectors]),
    ("fp8 dequant rounds once", "float v = orc_e4m3_decode(entry[i]) * sc[i / F8_GROUP];",
     "float v = " + ROUND_ONCE % "(double)orc_e4m3_decode(entry[i]) * (double)sc[i / F8_GROUP]" + ";",
     [ops.test_fp8_rounding_order_hand_vectors]),
    ("per-head scale as amax / (6 gs)", "uint8_t sf = orc_e4m3_encode((amax / 6.0f) / gs);",
     "uint8_t sf = orc_e4m3_encode(amax / (6.0f * gs));",
     [ops.test_perhead_hand_vectors]),
    ("per-head dequant rounds once", "o[i] = orc_f32_to_bf16_rne(code_times_scale * gs);",
     "o[i] = orc_f32_to_bf16_rne(" + ROUND_ONCE % "(double)code_times_scale * (double)gs" + ");",
     [ops.test_perhead_hand_vectors]),
]


def _build_mutant(tmp_path, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    (tmp_path / "gcache_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "gcache_oracle.h")).read())
    (tmp_path / "mutant.c").write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-fexcess-precision=standard", "-I", str(tmp_path), "-o", so, str(tmp_path / "mutant.c"),
                    "-lm"], check=True)
    return so


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pins):
    so = _build_mutant(tmp_path, old, new)
    good = oracle.lib()
    oracle._lib = oracle.lib(so)
    try:
        caught = 0
        for pin in pins:
            try:
                pin(oracle) if pin.__code__.co_argcount == 1 else pin(oracle, "nhd")
            except (AssertionError, oracle.OracleError):
                caught += 1
        assert caught > 0, f"no pin caught the planted mistake '{name}'"
    finally:
        oracle._lib = good
