"""Exhaustive check of the gfx950 conversion helpers the kernels use
(gather_concat_cache_amd/csrc/gcache_device.h) against the CPU oracle.

The writes round x * inv to e2m1 with v_cvt_scalef32_pk_fp4_f32 and to e4m3
with v_cvt_pk_fp8_f32 after a v_med3_f32 clamp; the gathers round binary32
products to bf16 with v_cvt_pk_bf16_f32; the scales come from binary32
divisions.  These stand in for the e2m1 pack of the vLLM PR #51724 digest's
write kernel ("Key source excerpts"), which rounds to nearest-even with
saturation.  Every binary32 pattern (NaNs excluded for the encoders) goes
through the device helpers in tests/pins/converter_sweep.hip, chunk by
chunk, and tests/pins/converter_check.c compares each result with the
oracle's encoders and with C's binary32 division.  Decoders are checked on
every code, and the general division of the per-head scale,
(amax / 6) / gs, on every positive finite bf16 amax against a sample of
per-tensor scales gs.

The CPU test at the end runs the host comparator on the oracle's own
outputs and on planted mismatches, so the GPU check cannot pass vacuously.
"""
import ctypes as C
import os

import numpy as np
import pytest
import torch

from conftest import ROOT

PINS = os.path.join(ROOT, "tests", "pins")
CHUNK = 1 << 26                      # binary32 patterns per device pass
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
WHAT = {1: "e2m1 code", 2: "e2m1 byte select", 3: "e4m3 code", 4: "bf16", 5: "x / 6", 6: "x / 448",
        7: "1 / x", 8: "(a / 6) / b"}


def _check_lib():
    path = os.path.join(PINS, "libconverter_check.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python tests/pins/build.py)")
    lib = C.CDLL(path)
    P, I64, U32 = C.c_void_p, C.c_int64, C.c_uint32
    lib.check_codes.argtypes = [U32, I64, P, P, P, C.c_int, C.POINTER(U32), C.POINTER(C.c_int)]
    lib.check_divs.argtypes = [U32, I64, P, P, P, C.c_int, C.POINTER(U32), C.POINTER(C.c_int)]
    lib.check_scale_div.argtypes = [P, P, P, I64, C.c_int, C.POINTER(U32), C.POINTER(C.c_int)]
    lib.check_decoders.argtypes = [P, P]
    for f in (lib.check_codes, lib.check_divs, lib.check_scale_div, lib.check_decoders):
        f.restype = I64
    return lib


def _sweep_lib():
    path = os.path.join(PINS, "libconverter_sweep.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python tests/pins/build.py)")
    lib = C.CDLL(path)
    P, U32 = C.c_void_p, C.c_uint32
    lib.sweep_unary.argtypes = [U32, U32, P, P, P, P, P, P, P]
    lib.sweep_scale_div.argtypes = [P, P, P, U32, P]
    lib.sweep_decoders.argtypes = [P, P, P]
    for f in (lib.sweep_unary, lib.sweep_scale_div, lib.sweep_decoders):
        f.restype = C.c_int
    return lib


def _ptr(a):
    return C.c_void_p(a.data_ptr() if isinstance(a, torch.Tensor) else a.ctypes.data)


def _report(bad, first, what, where):
    assert bad == 0, (f"{where}: {bad} mismatches; first at binary32 pattern {first.value:#010x} "
                      f"({WHAT.get(what.value, what.value)})")


# ---------------------------------------------------------------------------
@pytest.mark.gpu
def test_converters_every_binary32():
    """e2m1 (all four byte selectors), e4m3 with the saturating clamp, bf16
    rounding, x / 6, x / 448 and 1 / x on all 2^32 patterns."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sweep, check = _sweep_lib(), _check_lib()
    dev = {k: torch.empty(CHUNK * n, dtype=torch.uint8, device="cuda")
           for k, n in (("fp4", 1), ("fp8", 1), ("bf16", 2), ("div6", 4), ("div448", 4), ("recip", 4))}
    host = {k: torch.empty(v.numel(), dtype=torch.uint8, pin_memory=True) for k, v in dev.items()}
    stream = torch.cuda.current_stream().cuda_stream
    first, what = C.c_uint32(0), C.c_int(0)
    total = 0
    for base in range(0, 1 << 32, CHUNK):
        rc = sweep.sweep_unary(base, CHUNK, *(_ptr(dev[k]) for k in ("fp4", "fp8", "bf16", "div6", "div448",
                                                                    "recip")), C.c_void_p(stream))
        assert rc == 0, f"sweep launch failed ({rc}) at {base:#x}"
        for k in dev:
            host[k].copy_(dev[k], non_blocking=True)
        torch.cuda.synchronize()
        bad = check.check_codes(base, CHUNK, _ptr(host["fp4"]), _ptr(host["fp8"]), _ptr(host["bf16"]), THREADS,
                                C.byref(first), C.byref(what))
        _report(bad, first, what, "encoders")
        bad = check.check_divs(base, CHUNK, _ptr(host["div6"]), _ptr(host["div448"]), _ptr(host["recip"]),
                               THREADS, C.byref(first), C.byref(what))
        _report(bad, first, what, "divisions")
        total += CHUNK
    assert total == 1 << 32


@pytest.mark.gpu
def test_decoders_every_code():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sweep, check = _sweep_lib(), _check_lib()
    e4 = torch.zeros(256 * 5, dtype=torch.float32, device="cuda")
    e2 = torch.zeros(256 * 8, dtype=torch.float32, device="cuda")
    assert sweep.sweep_decoders(_ptr(e4), _ptr(e2), C.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    e4h, e2h = e4.cpu().numpy(), e2.cpu().numpy()
    assert check.check_decoders(_ptr(e4h), _ptr(e2h)) == 0


@pytest.mark.gpu
def test_perhead_scale_division():
    """(amax / 6) / gs for every positive finite bf16 amax (32639 values)
    against 2048 per-tensor scales: the harness's amax / 2688 family over
    ten decades plus random binary32 patterns in [2^-20, 2^10)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sweep, check = _sweep_lib(), _check_lib()
    amax = (np.arange(0x0001, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(2024)
    fam = (np.float32(10.0) ** rng.uniform(-5, 5, 1024).astype(np.float32)) / np.float32(2688.0)
    rnd = rng.integers(0x35800000, 0x44800000, 1024, dtype=np.uint32).view(np.float32)
    gs = np.concatenate([fam.astype(np.float32), rnd])
    a = np.repeat(amax, gs.size).astype(np.float32)
    b = np.tile(gs, amax.size).astype(np.float32)
    n = a.size
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    qd = torch.empty(n, dtype=torch.int32, device="cuda")
    assert sweep.sweep_scale_div(_ptr(ad), _ptr(bd), _ptr(qd), n,
                                 C.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    q = qd.cpu().numpy()
    first, what = C.c_uint32(0), C.c_int(0)
    bad = check.check_scale_div(_ptr(a), _ptr(b), _ptr(q), n, THREADS, C.byref(first), C.byref(what))
    _report(bad, first, what, "per-head scale division (index)")


# ---------------------------------------------------------------------------
def test_host_comparator_on_oracle_outputs_and_planted_mismatches(orc):
    """The comparator accepts the oracle's own results (laid out as the sweep
    kernel stores them) and reports a planted mismatch in each output."""
    check = _check_lib()
    base, n = 0x3E000000, 1 << 16                     # 0.125 .. about 0.5, plus the sign-free tail
    u = (base + np.arange(n, dtype=np.uint64)).astype(np.uint32)
    x = u.view(np.float32)
    e2 = orc.e2m1_encode(x)
    fp4 = np.empty(n, np.uint8)
    pair = (e2[0::2] | (e2[1::2] << 4)).astype(np.uint8)          # (x0, x1), (x2, x3) per word
    fp4[0::4], fp4[1::4], fp4[2::4], fp4[3::4] = pair[0::2], pair[1::2], pair[0::2], pair[1::2]
    fp8 = orc.e4m3_encode(x)
    bf = orc.f32_to_bf16(x)
    d6 = (x / np.float32(6)).view(np.uint32).copy()
    d448 = (x / np.float32(448)).view(np.uint32).copy()
    rc = (np.float32(1) / x).view(np.uint32).copy()
    first, what = C.c_uint32(0), C.c_int(0)
    args = lambda: (base, n, fp4.ctypes.data, fp8.ctypes.data, bf.ctypes.data, 4, C.byref(first), C.byref(what))
    dargs = lambda: (base, n, d6.ctypes.data, d448.ctypes.data, rc.ctypes.data, 4, C.byref(first), C.byref(what))
    assert check.check_codes(*args()) == 0 and check.check_divs(*dargs()) == 0
    for arr, k, fn, code in ((fp4, 4 * 100 + 2, check.check_codes, 2), (fp8, 777, check.check_codes, 3),
                             (bf, 5000, check.check_codes, 4), (d6, 123, check.check_divs, 5),
                             (rc, 4321, check.check_divs, 7)):
        arr[k] ^= 1
        got = fn(*(args() if fn is check.check_codes else dargs()))
        arr[k] ^= 1
        assert got >= 1 and what.value == code, (code, got, what.value)
    fp4[[4 * 7, 4 * 7 + 2]] ^= 0x10                                # odd element's nibble, both selectors
    assert check.check_codes(*args()) == 1 and what.value == 1 and first.value == base + 4 * 7 + 1
    fp4[[4 * 7, 4 * 7 + 2]] ^= 0x10
