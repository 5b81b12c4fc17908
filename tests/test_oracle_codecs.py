"""Pins of the oracle's scalar codecs against things other than itself.

* exhaustive: every binary32 pattern vs an independent rint-based encoder
  (tests/pins/codec_sweep.c);
* brute force: nearest-value search over every code (tests/brute.py) on all
  bf16 patterns and on binary32 values around every midpoint and grid value;
* library routines: torch's float8_e4m3fn and bfloat16 casts (round to
  nearest even) on in-range values, and torch's float8_e4m3fn decode;
* hand-derived vectors (tests/golden/e2m1_vectors.json, e4m3_vectors.json).
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import brute
from conftest import ROOT, load_golden


def _all_bf16_as_f32():
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)]


def _around_grid(mags, ulps=3):
    """binary32 values within +-ulps of every grid value and midpoint (both signs)."""
    pts = set(mags.tolist())
    pts |= {(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])}
    base = np.array(sorted(pts), dtype=np.float32).view(np.int32)
    offs = np.arange(-ulps, ulps + 1, dtype=np.int32)
    u = (base[:, None] + offs[None, :]).ravel()
    u = u[u >= 0]
    f = u.view(np.float32)
    return np.concatenate([f, -f])


def test_decoders_match_format_tables(orc):
    # e2m1: the OCP MX E2M1 value table
    codes = np.arange(16, dtype=np.uint8)
    want = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 2) * np.repeat([1, -1], 8)
    got = orc.e2m1_decode(codes)
    assert np.array_equal(got, want.astype(np.float32))
    assert np.array_equal(np.signbit(got[8]), True)          # 0x8 is -0
    # e4m3: torch's float8_e4m3fn decode (an independent implementation)
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = orc.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


@pytest.mark.parametrize("which", ["e2m1", "e4m3"])
def test_encoders_match_nearest_value_brute_force(orc, which):
    mags = brute.E2M1_MAG if which == "e2m1" else brute.E4M3_MAG
    rng = np.random.default_rng(7)
    y = np.concatenate([
        _all_bf16_as_f32(),
        _around_grid(mags),
        rng.standard_normal(200_000).astype(np.float32) * np.float32(4 if which == "e2m1" else 200),
        (rng.random(200_000, dtype=np.float32) - np.float32(0.5)) * np.float32(2.0 ** -6),
    ]).astype(np.float32)
    enc = orc.e2m1_encode if which == "e2m1" else orc.e4m3_encode
    bf = brute.e2m1_encode if which == "e2m1" else brute.e4m3_encode
    got, want = enc(y), bf(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{which}: {bad.size} mismatches, first y={y[bad[0]]!r} got {got[bad[0]]:#x} want {want[bad[0]]:#x}"


def test_e4m3_encoder_matches_torch_cast_in_range(orc):
    """torch's float8_e4m3fn cast rounds to nearest even but does not saturate:
    compare where |y| < 464 (below the first value that would round past 448)."""
    rng = np.random.default_rng(11)
    y = np.concatenate([_all_bf16_as_f32(), _around_grid(brute.E4M3_MAG),
                        rng.standard_normal(500_000).astype(np.float32) * np.float32(100)])
    y = y[np.abs(y) < 464].astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_encode(y)
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch_cast(orc):
    """Every bf16 pattern with low halves at and around the tie point."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    y = u.view(np.float32)
    y = y[np.isfinite(y)]
    ref = torch.from_numpy(y.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f32_to_bf16(y)
    finite = np.isfinite(torch.from_numpy(y.copy()).to(torch.bfloat16).float().numpy())
    assert np.array_equal(got[finite], ref[finite])
    # overflow rounds to infinity like torch
    assert np.array_equal(got[~finite], ref[~finite])
    # the independent neighbour-choice formulation agrees too
    assert np.array_equal(got, brute.to_bf16_bits(y))


def test_hand_vectors(orc):
    for name, enc in (("e2m1_vectors.json", orc.e2m1_encode), ("e4m3_vectors.json", orc.e4m3_encode)):
        cases = load_golden(name)["cases"]
        y = np.array([c["x"] for c in cases], dtype=np.float32)
        want = np.array([int(c["code"], 16) for c in cases], dtype=np.uint8)
        got = enc(y)
        for c, g, w in zip(cases, got, want):
            assert g == w, f"{name}: {c['x']} -> {g:#x}, expected {w:#x} ({c['why']})"


@pytest.mark.slow
def test_exhaustive_sweep_against_independent_encoder(tmp_path):
    """All 2^32 binary32 patterns: oracle e2m1 / e4m3 / bf16 vs rint-based
    formulations (tests/pins/codec_sweep.c).  About 30 s on 8 cores."""
    exe = str(tmp_path / "codec_sweep")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-o", exe,
                    os.path.join(ROOT, "tests", "pins", "codec_sweep.c"),
                    os.path.join(ROOT, "oracle", "gcache_oracle.c"), "-lm", "-lpthread"], check=True)
    threads = str(min(16, os.cpu_count() or 8))
    out = subprocess.run([exe, threads], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout


def test_sweep_checker_detects_a_planted_error(tmp_path):
    """The sweep fails when the oracle's e4m3 tie rule is flipped (a mutant
    oracle built on the CPU): the sweep is not vacuous."""
    src = open(os.path.join(ROOT, "oracle", "gcache_oracle.c")).read()
    mutant = src.replace("return (lo % 2 == 0) ? lo : hi;", "return (lo % 2 == 0) ? hi : lo;")
    assert mutant != src
    (tmp_path / "gcache_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "gcache_oracle.h")).read())
    (tmp_path / "mutant.c").write_text(mutant)
    exe = str(tmp_path / "sweep_mutant")
    sweep = open(os.path.join(ROOT, "tests", "pins", "codec_sweep.c")).read()
    (tmp_path / "sweep.c").write_text(sweep.replace('#include "../../oracle/gcache_oracle.h"',
                                                    '#include "gcache_oracle.h"'))
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-I", str(tmp_path), "-o", exe,
                    str(tmp_path / "sweep.c"), str(tmp_path / "mutant.c"), "-lm", "-lpthread"],
                   check=True)
    # 1.0625 = 0x3F880000 is an e4m3 tie; sweep a small range around it
    out = subprocess.run([exe, "2", "3f870000", "3f890000"], capture_output=True, text=True)
    assert out.returncode == 1 and "e4m3 mismatch" in out.stdout
