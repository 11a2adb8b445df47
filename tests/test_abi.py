"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
its host-only plan matches the oracle's closed form, and every argument
check fails before anything reaches the device (no GPU is needed: each call
below is rejected by host validation or is an empty request)."""

import ctypes
import os
import random
import re

import pytest

from oracle import plan as OP
import serving_sk_score_amd.sk as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sk.h")

# tests/test_host_sanitize.py runs this module in a child process whose
# SK_ABI_TEST_LIB names a host-sanitized build of the same sources; every
# call below then goes through that build.
if os.environ.get("SK_ABI_TEST_LIB"):
    sk._lib = sk.bind(os.environ["SK_ABI_TEST_LIB"])


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sk_[a-z_0-9]+)\s*\(", text)) - {"sk_status"})


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 12
    lib = sk.lib()
    for nm in names:
        assert hasattr(lib, nm), nm
    assert set(names) == set(sk.EXPORTS)


def test_layout_version_and_strings():
    lib = sk.lib()
    assert lib.sk_layout_version() == 1
    for st in range(6):
        assert lib.sk_status_string(st)
    assert b"unknown" in lib.sk_status_string(99)


def _oracle_or_err(L, Hq, H, d, n, S, b, three, overflow=0):
    try:
        return OP.make_plan(L, Hq, H, d, n, S, b, three, overflow)
    except OP.BudgetError:
        return "budget"


def test_plan_parity_random():
    rnd = random.Random(1)
    shapes = [(1, 4, 2, 64), (32, 32, 8, 128), (28, 28, 4, 128), (42, 16, 8, 256), (3, 7, 7, 64)]
    for _ in range(4000):
        L, Hq, H, d = rnd.choice(shapes)
        n = rnd.choice([0, 1, 2, 3, 5, 17, 255, 256, 1000, 8192, 32768, 65536, rnd.randint(0, 200000)])
        S = rnd.choice([0, 1, 4, 32])
        b = rnd.choice([0.0, 0.25, 0.3, 0.5, 0.6, 0.7, 1.0, round(rnd.random(), 4)])
        three = rnd.choice([0, 1])
        mode = rnd.choice([sk.OVERFLOW_REJECT, sk.OVERFLOW_DROP, sk.OVERFLOW_FALLBACK])
        assert (OP.REJECT, OP.DROP_OVERFLOW, OP.FALLBACK) == (0, 1, 2)
        want = _oracle_or_err(L, Hq, H, d, n, S, b, three, mode)
        pol = sk.Policy(n, S, three, b, mode)
        if want == "budget":
            with pytest.raises(sk.SkError) as e:
                sk.plan_make(sk.Shape(L, Hq, H, d), pol)
            assert e.value.status == sk.SK_E_BUDGET
            continue
        got = sk.plan_make(sk.Shape(L, Hq, H, d), pol)
        for f in ("n16", "n8", "n4", "n_drop", "budget_units", "used_units", "payload_bytes",
                  "off_c16", "off_c8", "off_c4", "off_s8", "off_s4"):
            assert getattr(got, f) == getattr(want, f), (f, L, Hq, H, d, n, S, b, three, mode)
        assert got.n_sink == want.sinks


@pytest.mark.parametrize("shape,policy,status", [
    ((1, 4, 2, 96), (10, 0, 1, 0.5), sk.SK_E_UNSUPPORTED),
    ((1, 3, 2, 64), (10, 0, 1, 0.5), sk.SK_E_ARG),
    ((0, 4, 2, 64), (10, 0, 1, 0.5), sk.SK_E_ARG),
    ((1, 34, 2, 64), (10, 0, 1, 0.5), sk.SK_E_UNSUPPORTED),
    ((1, 4, 2, 64), (-1, 0, 1, 0.5), sk.SK_E_ARG),
    ((1, 4, 2, 64), (1 << 30, 0, 1, 0.5), sk.SK_E_ARG),
    ((1, 4, 2, 64), (10, -1, 1, 0.5), sk.SK_E_ARG),
    ((1, 4, 2, 64), (10, 0, 2, 0.5), sk.SK_E_ARG),
    ((1, 4, 2, 64), (10, 0, 1, 1.5), sk.SK_E_ARG),
    ((1, 4, 2, 64), (10, 0, 1, float("nan")), sk.SK_E_ARG),
    ((1, 4, 2, 64), (1000, 0, 1, 0.2), sk.SK_E_BUDGET),
    ((1, 4, 2, 64), (256, 4, 0, 0.5), sk.SK_E_BUDGET),
    ((1, 4, 2, 64), (10, 0, 1, 0.5, 3), sk.SK_E_ARG),
    ((1, 4, 2, 64), (100, 30, 1, 0.2, 1), sk.SK_E_BUDGET),     # drop mode: sinks overrun
])
def test_plan_failures(shape, policy, status):
    with pytest.raises(sk.SkError) as e:
        sk.plan_make(sk.Shape(*shape), sk.Policy(*policy))
    assert e.value.status == status
    assert sk.lib().sk_last_error()


def _c(shape, policy=None):
    s = sk.Shape(*shape).c()
    p = sk.Policy(*policy).c() if policy else None
    return s, p


def _plan(shape, policy):
    return sk.plan_make(sk.Shape(*shape), sk.Policy(*policy))


FAKE = ctypes.c_void_p(0x7F0000001000)       # never dereferenced: every call below fails first
FAKE_MIS = ctypes.c_void_p(0x7F0000001002)   # misaligned


def test_call_validation_without_device():
    lib = sk.lib()
    B = ctypes.byref
    shape, pol = _c((2, 4, 2, 64), (100, 4, 1, 0.5))
    plan = _plan((2, 4, 2, 64), (100, 4, 1, 0.5))
    pc = plan.c
    # score: NULL pointers, misalignment, workspace too small
    assert lib.sk_score(B(shape), 100, None, FAKE, FAKE, 0, FAKE, 1 << 20, None) == sk.SK_E_ARG
    assert lib.sk_score(B(shape), 100, FAKE_MIS, FAKE, FAKE, 0, FAKE, 1 << 20, None) == sk.SK_E_ARG
    need = lib.sk_score_workspace_bytes(B(shape), 100)
    assert need > 0
    assert lib.sk_score(B(shape), 100, FAKE, FAKE, FAKE, 0, FAKE, need - 1, None) == sk.SK_E_WORKSPACE
    assert lib.sk_score(B(shape), 100, FAKE, FAKE, FAKE, 2, FAKE, need, None) == sk.SK_E_ARG
    assert lib.sk_score_colsum(B(shape), 100, FAKE, FAKE, FAKE, FAKE, 0, None, 0, None) == sk.SK_E_WORKSPACE
    assert lib.sk_score_rowlse(B(shape), 100, FAKE, FAKE, None, None) == sk.SK_E_ARG
    bad_shape, _ = _c((2, 4, 2, 80))
    assert lib.sk_score(B(bad_shape), 100, FAKE, FAKE, FAKE, 0, FAKE, need, None) == sk.SK_E_UNSUPPORTED
    # longer than the launch grid of the row pass holds (65535 blocks of 64)
    big = 65535 * 64 + 1
    assert lib.sk_score_rowlse(B(shape), big, FAKE, FAKE, FAKE, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score(B(shape), big, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_workspace_bytes(B(shape), big) == 0
    assert lib.sk_score_colsum_workspace_bytes(B(shape), big) == 0
    assert lib.sk_score_workspace_bytes(B(shape), big - 1) > 0
    # allocation-free score: same argument checks, and a request larger than
    # the static scratch is rejected before any device is touched
    assert lib.sk_score_noalloc(B(shape), 100, None, FAKE, FAKE, 0, None) == sk.SK_E_ARG
    assert lib.sk_score_noalloc(B(shape), 100, FAKE, FAKE, FAKE, 2, None) == sk.SK_E_ARG
    assert lib.sk_score_noalloc(B(bad_shape), 100, FAKE, FAKE, FAKE, 0, None) == sk.SK_E_UNSUPPORTED
    wide, _ = _c((1, 32, 8, 128))
    for n_big in (131073, 1 << 20):
        assert lib.sk_score_workspace_bytes(B(wide), n_big) > sk.SCORE_SCRATCH_BYTES
        assert lib.sk_score_noalloc(B(wide), n_big, FAKE, FAKE, FAKE, 0, None) == sk.SK_E_WORKSPACE
        assert b"scratch" in lib.sk_last_error()
    assert lib.sk_score_workspace_bytes(B(wide), 131072) == sk.SCORE_SCRATCH_BYTES
    assert lib.sk_score_noalloc(B(shape), 0, None, None, None, 0, None) == sk.SK_OK
    # empty request: OK and nothing touched even with NULL buffers
    assert lib.sk_score(B(shape), 0, None, None, None, 0, None, 0, None) == sk.SK_OK
    assert lib.sk_score_rowlse(B(shape), 0, None, None, None, None) == sk.SK_OK
    # all-layer score: the same argument rules, an L-fold workspace, and a
    # layer count the launch grid cannot hold is refused
    lneed = lib.sk_score_layers_workspace_bytes(B(shape), 100)
    assert lneed == 2 * need
    assert lib.sk_score_colsum_layers_workspace_bytes(B(shape), 100) == \
        2 * lib.sk_score_colsum_workspace_bytes(B(shape), 100)
    assert lib.sk_score_layers(B(shape), 100, None, FAKE, FAKE, 0, FAKE, lneed, None) == sk.SK_E_ARG
    assert lib.sk_score_layers(B(shape), 100, FAKE, FAKE, FAKE, 2, FAKE, lneed, None) == sk.SK_E_ARG
    assert lib.sk_score_layers(B(shape), 100, FAKE, FAKE, FAKE, 0, FAKE, lneed - 1, None) == sk.SK_E_WORKSPACE
    assert lib.sk_score_layers(B(shape), 100, FAKE, FAKE, FAKE, 0, FAKE_MIS, lneed, None) == sk.SK_E_ARG
    assert lib.sk_score_layers(B(bad_shape), 100, FAKE, FAKE, FAKE, 0, FAKE, lneed, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_rowlse_layers(B(shape), 100, FAKE, FAKE, None, None) == sk.SK_E_ARG
    assert lib.sk_score_rowlse_layers(B(shape), big, FAKE, FAKE, FAKE, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_colsum_layers(B(shape), 100, FAKE, FAKE, FAKE, FAKE, 0, None, 0, None) == sk.SK_E_WORKSPACE
    assert lib.sk_score_colsum_layers(B(shape), 100, FAKE, FAKE, None, FAKE, 0, FAKE, lneed, None) == sk.SK_E_ARG
    # a workspace that n_layers times the one-layer size would overflow
    huge, _ = _c((65535, 16 * (2 ** 27 - 1), 2 ** 27 - 1, 64))
    assert lib.sk_score_layers_workspace_bytes(B(huge), 4_000_000) == 0
    assert lib.sk_score_colsum_layers_workspace_bytes(B(huge), 4_000_000) == 0
    assert lib.sk_score_layers(B(huge), 4_000_000, FAKE, FAKE, FAKE, 0, FAKE, 1 << 62, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_colsum_layers(B(huge), 4_000_000, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 62, None) == sk.SK_E_UNSUPPORTED
    assert b"overflows" in lib.sk_last_error()
    assert lib.sk_score_workspace_bytes(B(huge), 4_000_000) > 0   # one layer still fits
    deep, _ = _c((65536, 4, 2, 64))
    assert lib.sk_score_layers_workspace_bytes(B(deep), 100) == 0
    assert lib.sk_score_layers(B(deep), 100, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_rowlse_layers(B(deep), 100, FAKE, FAKE, FAKE, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_layers(B(shape), 0, None, None, None, 0, None, 0, None) == sk.SK_OK
    assert lib.sk_score_rowlse_layers(B(shape), 0, None, None, None, None) == sk.SK_OK
    assert lib.sk_score_colsum_layers(B(shape), 0, None, None, None, None, 0, None, 0, None) == sk.SK_OK
    # assign: plan / policy disagreement, NULLs
    other = sk.Policy(101, 4, 1, 0.5).c()
    assert lib.sk_assign_tiers(B(other), B(pc), FAKE, FAKE, FAKE, None, 0, None) == sk.SK_E_ARG
    assert lib.sk_assign_tiers(B(pol), B(pc), None, FAKE, FAKE, None, 0, None) == sk.SK_E_ARG
    # pack / unpack: corrupted plan, shape mismatch, misaligned payload
    bad = sk._Plan.from_buffer_copy(pc)
    bad.n8 += 1
    # decode attention: layer range, NULLs, alignment, workspace
    dws = lib.sk_decode_workspace_bytes(B(shape), B(pc), 2)
    assert dws > 0 and lib.sk_decode_workspace_bytes(B(shape), B(pc), 3) == 0
    assert lib.sk_decode_attention(B(shape), B(pc), FAKE, 1, 2, FAKE, FAKE, None, FAKE, dws, None) == sk.SK_E_ARG
    assert lib.sk_decode_attention(B(shape), B(pc), FAKE, 0, 0, FAKE, FAKE, None, FAKE, dws, None) == sk.SK_E_ARG
    assert lib.sk_decode_attention(B(shape), B(pc), FAKE, 0, 2, None, FAKE, None, FAKE, dws, None) == sk.SK_E_ARG
    assert lib.sk_decode_attention(B(shape), B(pc), FAKE, 0, 2, FAKE_MIS, FAKE, None, FAKE, dws, None) == sk.SK_E_ARG
    assert lib.sk_decode_attention(B(shape), B(pc), FAKE, 0, 2, FAKE, FAKE, None, FAKE, dws - 1, None) == sk.SK_E_WORKSPACE
    assert lib.sk_decode_attention(B(shape), B(bad), FAKE, 0, 2, FAKE, FAKE, None, FAKE, dws, None) == sk.SK_E_ARG
    assert lib.sk_decode_attention(B(shape), B(pc), ctypes.c_void_p(0x7F0000001010), 0, 2, FAKE, FAKE, None, FAKE, dws, None) == sk.SK_E_ARG
    # more KV heads than a decode launch grid holds
    wide_kv = (1, 65536, 65536, 64)
    wpc = _plan(wide_kv, (100, 4, 1, 0.5)).c
    wshape, _ = _c(wide_kv)
    assert lib.sk_decode_workspace_bytes(B(wshape), B(wpc), 1) == 0
    assert lib.sk_decode_attention(B(wshape), B(wpc), FAKE, 0, 1, FAKE, FAKE, None, FAKE, 1 << 40, None) == sk.SK_E_UNSUPPORTED
    ok_kv = (1, 65535, 65535, 64)
    assert lib.sk_decode_workspace_bytes(B(_c(ok_kv)[0]), B(_plan(ok_kv, (100, 4, 1, 0.5)).c), 1) > 0
    assert lib.sk_pack(B(shape), B(bad), FAKE, FAKE, FAKE, None, FAKE, None) == sk.SK_E_ARG
    shape2, _ = _c((3, 4, 2, 64))
    assert lib.sk_pack(B(shape2), B(pc), FAKE, FAKE, FAKE, None, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_pack(B(shape), B(pc), FAKE, FAKE, FAKE, None, ctypes.c_void_p(0x7F0000001010), None) == sk.SK_E_ARG
    assert lib.sk_pack(B(shape), B(pc), FAKE, None, FAKE, None, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_unpack(B(shape), B(pc), FAKE, FAKE, None, FAKE, None, None) == sk.SK_E_ARG
    pg = sk._Paged(0x7F0000001000, 0x7F0000001000, 0x7F0000001000, 16, 3)  # needs 7 blocks
    assert lib.sk_unpack(B(shape), B(pc), FAKE, FAKE, None, None, B(pg), None) == sk.SK_E_ARG
    pg0 = sk._Paged(0x7F0000001000, 0x7F0000001000, 0x7F0000001000, 0, 7)
    assert lib.sk_unpack(B(shape), B(pc), FAKE, FAKE, None, None, B(pg0), None) == sk.SK_E_ARG
    assert lib.sk_unpack(B(shape), B(pc), FAKE, FAKE, FAKE, FAKE, B(pg), None) == sk.SK_E_ARG
    # score variants: lambda out of range, overlap, NULLs, accumulate flag
    assert lib.sk_recency_weight(10, -0.5, FAKE, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_recency_weight(10, float("nan"), FAKE, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_recency_weight(10, 0.5, None, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_recency_weight(10, 0.5, FAKE, ctypes.c_void_p(0x7F0000001008), None) == sk.SK_E_ARG
    assert lib.sk_recency_weight(-1, 0.5, FAKE, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_recency_weight(0, 0.5, None, None, None) == sk.SK_OK
    assert lib.sk_score_kvnorm(B(shape), 10, None, FAKE, 0, None) == sk.SK_E_ARG
    assert lib.sk_score_kvnorm(B(shape), 10, FAKE_MIS, FAKE, 0, None) == sk.SK_E_ARG
    assert lib.sk_score_kvnorm(B(shape), 10, FAKE, FAKE, 2, None) == sk.SK_E_ARG
    assert lib.sk_score_kvnorm(B(bad_shape), 10, FAKE, FAKE, 0, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_score_kvnorm(B(shape), 0, None, None, 0, None) == sk.SK_OK
    # balanced keys
    assert lib.sk_balanced_keys(10, 2, None, None) == sk.SK_E_ARG
    assert lib.sk_balanced_keys(10, -2, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_balanced_keys((1 << 24) + 5, 4, FAKE, None) == sk.SK_E_UNSUPPORTED
    assert lib.sk_balanced_keys(0, 0, None, None) == sk.SK_OK
    # upgrade: sizes, NULLs, alignment, paged argument rules
    assert lib.sk_upgrade_bytes(B(shape), 3) == 2 * 3 * 2 * 2 * 2 * 64
    assert lib.sk_upgrade_bytes(B(shape), -1) == 0
    assert lib.sk_upgrade_bytes(B(bad_shape), 3) == 0
    assert lib.sk_upgrade_pack(B(shape), 100, FAKE, FAKE, None, 3, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_upgrade_pack(B(shape), 100, FAKE, FAKE, FAKE, 3, FAKE_MIS, None) == sk.SK_E_ARG
    assert lib.sk_upgrade_pack(B(shape), 100, FAKE, FAKE, FAKE, -3, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_upgrade_pack(B(shape), 100, None, FAKE, FAKE, 3, FAKE, None) == sk.SK_E_ARG
    assert lib.sk_upgrade_pack(B(shape), 100, None, None, None, 0, None, None) == sk.SK_OK
    assert lib.sk_upgrade_unpack(B(shape), 100, FAKE, FAKE, 3, FAKE, None, None, None) == sk.SK_E_ARG
    assert lib.sk_upgrade_unpack(B(shape), 100, FAKE, FAKE, 3, FAKE, FAKE, B(pg), None) == sk.SK_E_ARG
    pg_ok = sk._Paged(0x7F0000001000, 0x7F0000001000, 0x7F0000001002, 16, 7)
    assert lib.sk_upgrade_unpack(B(shape), 100, FAKE, FAKE, 3, None, None, B(pg_ok), None) == sk.SK_E_ARG
    assert lib.sk_upgrade_unpack(B(shape), 100, FAKE, FAKE, 3, None, None, B(pg), None) == sk.SK_E_ARG
    assert lib.sk_upgrade_unpack(B(shape), 100, None, None, 0, None, None, None, None) == sk.SK_OK
    # shapes whose fp16 KV would pass 2^62 bytes: no plan, no upgrade size
    vast, _ = _c((65535, 2 ** 30, 2 ** 26, 256))
    vp = sk.Policy(1 << 20, 4, 1, 0.5).c()
    assert lib.sk_plan_make(B(vast), B(vp), B(sk._Plan())) == sk.SK_E_UNSUPPORTED
    assert b"2^62" in lib.sk_last_error()
    assert lib.sk_upgrade_bytes(B(vast), 1 << 20) == 0
    assert lib.sk_upgrade_pack(B(vast), 1 << 20, FAKE, FAKE, FAKE, 3, FAKE, None) == sk.SK_E_UNSUPPORTED
    empty = _plan((2, 4, 2, 64), (0, 4, 1, 0.5))
    assert lib.sk_pack(B(shape), B(empty.c), None, None, None, None, None, None) == sk.SK_OK
    assert lib.sk_unpack(B(shape), B(empty.c), None, None, None, None, None, None) == sk.SK_OK


def test_workspace_sizes():
    lib = sk.lib()
    B = ctypes.byref
    for shp, n in [((1, 4, 2, 64), 256), ((32, 32, 8, 128), 8192), ((42, 16, 8, 256), 32768)]:
        s = sk.Shape(*shp).c()
        total = lib.sk_score_workspace_bytes(B(s), n)
        col = lib.sk_score_colsum_workspace_bytes(B(s), n)
        assert total >= col + shp[1] * n * 4 and col >= 4 * n
    assert lib.sk_score_workspace_bytes(B(sk.Shape(1, 4, 2, 96).c()), 10) == 0
