"""The C ABI library loads and exports what include/base_layer.h declares;
host-side argument checks and workspace sizing run without a GPU (no kernel
is launched on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

from balanced_token_expert_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "base_layer.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char \*|size_t |int )\s*(base_\w+)\s*\(", src,
                                 re.M)))


def test_phase_events_arg_check(lib):
    assert lib.base_set_phase_events(None, 0) == 0
    assert lib.base_set_phase_events(None, 9) == api.BASE_ERR_INVALID_ARG
    assert lib.base_set_auction_events(None, 0) == 0
    assert lib.base_set_auction_events(None, 64) == 0
    assert lib.base_set_auction_events(None, 65) == api.BASE_ERR_INVALID_ARG
    assert lib.base_set_auction_events(None, -1) == api.BASE_ERR_INVALID_ARG


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        import balanced_token_expert_amd.build as b
        b.build()
    return api.load()


def test_header_declares_the_entry_points():
    assert _declared() == sorted(api.EXPORTED)


def test_checking_build_exports_every_declared_symbol(lib):
    """The checking variant (BASE_CHECKS) exposes the same C ABI."""
    import balanced_token_expert_amd.build as b
    assert os.path.exists(b.LIB_CHECKS), "libbase_layer_checks.so not built"
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_CHECKS], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (base_\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (base_\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_strerror(lib):
    assert api.strerror(0) == "ok"
    assert "multiple" in api.strerror(api.BASE_ERR_INDIVISIBLE)
    assert api.strerror(12345) == "unknown error"


def test_workspace_sizes(lib):
    T, E, D, F = 65536, 128, 2048, 8192
    lay = api.base_workspace_bytes(api.BASE_OP_LAYER, T, E, D, F, api.BASE_BF16)
    # the hidden activations (T x F bf16) and the scores dominate, then the
    # phase end's expert-major copy of the holders' scores (T x E fp32, for
    # E <= 128); the rest is per-token bookkeeping and per-expert scratch
    # (the auction's bid bins take 40 KiB per expert)
    assert lay >= T * F * 2 + 2 * T * E * 4
    assert lay < T * F * 2 + 2 * T * E * 4 + 64 * T + 48 * 1024 * E + (1 << 20)
    auc = api.base_workspace_bytes(api.BASE_OP_AUCTION, T, E)
    assert 0 < auc < lay
    assert api.base_workspace_bytes(api.BASE_OP_AFFINITY, T, E, D) == 0
    assert api.base_workspace_bytes(api.BASE_OP_LAYER, 0, E, D, F) == 0


def _auction(lib, T, E, c, ws_bytes=1 << 30):
    return lib.base_assign_auction(FAKE, T, E, c, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_bytes,
                                   None)


def test_auction_host_errors(lib):
    good = api.cfg(1.0, 1e-4, 10.0, 0)
    assert _auction(lib, 10, 3, good) == api.BASE_ERR_INDIVISIBLE
    assert _auction(lib, 4, 8, good) == api.BASE_ERR_INVALID_ARG         # E > T
    assert _auction(lib, 0, 1, good) == api.BASE_ERR_INVALID_ARG
    assert _auction(lib, 12, 3, api.cfg(1e-4, 1.0)) == api.BASE_ERR_INVALID_ARG
    assert _auction(lib, 12, 3, api.cfg(1.0, 0.0)) == api.BASE_ERR_INVALID_ARG
    assert _auction(lib, 12, 3, api.cfg(1.0, 1e-4, 1.0)) == api.BASE_ERR_INVALID_ARG
    assert _auction(lib, 12, 3, api.cfg(1e30, 1e-30, 1.5)) == api.BASE_ERR_INVALID_ARG
    assert _auction(lib, 12, 3, good, ws_bytes=16) == api.BASE_ERR_INVALID_ARG
    assert _auction(lib, 2048 * 2048, 2048, good) == api.BASE_ERR_UNSUPPORTED  # E > 1024
    assert lib.base_assign_auction(None, 12, 3, good, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   1 << 30, None) == api.BASE_ERR_INVALID_ARG


def test_greedy_noalloc_host_errors(lib):
    # beyond the static 8 MiB scratch, and the usual argument checks; all
    # refused before anything is enqueued
    assert lib.base_route_greedy_noalloc(FAKE, 1 << 24, 128, FAKE, FAKE, FAKE, FAKE, None) == \
        api.BASE_ERR_UNSUPPORTED
    assert lib.base_route_greedy_noalloc(None, 16, 4, FAKE, None, None, None, None) == \
        api.BASE_ERR_INVALID_ARG
    assert lib.base_route_greedy_noalloc(FAKE, 16, 4, FAKE, None, FAKE, None, None) == \
        api.BASE_ERR_INVALID_ARG
    assert lib.base_route_greedy_noalloc(FAKE, 16, 8192, FAKE, FAKE, None, None, None) == \
        api.BASE_ERR_UNSUPPORTED


def test_layer_host_errors(lib):
    good = api.cfg(1.0, 1e-4, 10.0, 0)

    def call(T=12, E=3, D=8, F=16, dt=1, act=1, mode=0, c=good, ws=1 << 30, ptr=FAKE):
        return lib.base_layer_forward(ptr, FAKE, FAKE, FAKE, T, E, D, F, dt, act, mode, c, FAKE,
                                      None, None, FAKE, None, FAKE, ws, None)

    assert call(T=10) == api.BASE_ERR_INDIVISIBLE
    # greedy routing has ragged groups: T % E need not be 0 (here the
    # workspace check is what fails)
    assert call(T=10, mode=api.BASE_ROUTE_GREEDY, ws=1) == api.BASE_ERR_INVALID_ARG
    assert call(mode=7) == api.BASE_ERR_INVALID_ARG
    assert call(act=5) == api.BASE_ERR_INVALID_ARG
    assert call(dt=9) == api.BASE_ERR_INVALID_ARG
    assert call(F=0) == api.BASE_ERR_INVALID_ARG
    assert call(D=12) == api.BASE_ERR_UNSUPPORTED            # bf16 needs D % 8 == 0
    assert call(ws=100) == api.BASE_ERR_INVALID_ARG
    assert call(ptr=None) == api.BASE_ERR_INVALID_ARG
    assert call(c=api.cfg(1e-4, 1e-2)) == api.BASE_ERR_INVALID_ARG


def test_greedy_and_affinity_host_errors(lib):
    assert lib.base_route_greedy(FAKE, 0, 3, FAKE, None, None, None, FAKE, 1 << 20,
                                 None) == api.BASE_ERR_INVALID_ARG
    assert lib.base_route_greedy(FAKE, 12, 3, FAKE, None, FAKE, None, FAKE, 1 << 20,
                                 None) == api.BASE_ERR_INVALID_ARG   # perm without offsets
    assert lib.base_route_greedy(FAKE, 12, 3, FAKE, None, None, None, FAKE, 8,
                                 None) == api.BASE_ERR_INVALID_ARG   # workspace too small
    # more experts than the grouping kernels hold: refused on the host when
    # counts or the grouping are asked for (nothing is launched)
    big = api.base_workspace_bytes(api.BASE_OP_GREEDY, 8192, 8192, 0, 0, 0)
    assert big > 0
    assert lib.base_route_greedy(FAKE, 8192, 8192, FAKE, FAKE, None, None, FAKE, big,
                                 None) == api.BASE_ERR_UNSUPPORTED   # counts
    assert lib.base_route_greedy(FAKE, 8192, 8192, FAKE, None, FAKE, FAKE, FAKE, big,
                                 None) == api.BASE_ERR_UNSUPPORTED   # perm + offsets
    assert lib.base_affinity(FAKE, FAKE, None, 12, 3, 8, 1, None) == api.BASE_ERR_INVALID_ARG
    assert lib.base_affinity(FAKE, FAKE, FAKE, 12, 3, 12, 1, None) == api.BASE_ERR_UNSUPPORTED
    assert lib.base_affinity(FAKE, FAKE, FAKE, 12, 3, 8, 4, None) == api.BASE_ERR_INVALID_ARG


def test_layer_ex_host_errors(lib):
    good = api.cfg(1.0, 1e-4, 10.0, 0)
    T, E, D, F = 12, 3, 8, 16
    lay = api.base_workspace_bytes(api.BASE_OP_LAYER, T, E, D, F, api.BASE_BF16)
    lay_ex = api.base_workspace_bytes(api.BASE_OP_LAYER_EX, T, E, D, F, api.BASE_BF16)
    assert lay_ex >= lay + 2 * T * D * 2

    def call(mix=0, sub=1, eps=1e-5, ws=1 << 30, T=T):
        o = api.LayerOpts(mix, sub, eps, None, None)
        return lib.base_layer_forward_ex(FAKE, FAKE, FAKE, FAKE, T, E, D, F, 1, 1, 0, good, FAKE,
                                         None, None, FAKE, None, ctypes.byref(o), FAKE, ws, None)

    assert call(mix=2) == api.BASE_ERR_INVALID_ARG
    assert call(sub=-1) == api.BASE_ERR_INVALID_ARG
    assert call(sub=65) == api.BASE_ERR_INVALID_ARG
    assert call(eps=-1.0) == api.BASE_ERR_INVALID_ARG
    assert call(ws=lay) == api.BASE_ERR_INVALID_ARG        # needs the LAYER_EX workspace
    assert call(T=10) == api.BASE_ERR_INDIVISIBLE


def test_backward_host_errors(lib):
    T, E, D, F = 12, 3, 8, 16
    bf = api.BASE_BF16
    ws_plain = api.base_workspace_bytes(api.BASE_OP_LAYER_BWD, T, E, D, F, bf)

    def call(T=T, D=D, F=F, dt=1, act=1, mix=0, sub=None, eps=1e-5, ws=1 << 30, ex=False,
             ptr=FAKE):
        o = None if sub is None else api.LayerOpts(mix, sub, eps, None, None)
        op = None if o is None else ctypes.byref(o)
        args = [ptr, FAKE, FAKE, FAKE, T, E, D, F, dt, act, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                FAKE]
        if ex:
            return lib.base_layer_backward_ex(*args, None, None, None, op, FAKE, ws, None)
        return lib.base_layer_backward(*args, None, op, FAKE, ws, None)

    for ex in (False, True):
        assert call(ptr=None, ex=ex) == api.BASE_ERR_INVALID_ARG
        assert call(T=0, ex=ex) == api.BASE_ERR_INVALID_ARG
        assert call(dt=9, ex=ex) == api.BASE_ERR_INVALID_ARG
        assert call(act=5, ex=ex) == api.BASE_ERR_INVALID_ARG
        assert call(mix=2, sub=0, ex=ex) == api.BASE_ERR_INVALID_ARG
        assert call(D=12, ex=ex) == api.BASE_ERR_UNSUPPORTED          # bf16 needs D % 8 == 0
        assert call(F=(1 << 20) + 8, ex=ex) == api.BASE_ERR_UNSUPPORTED  # 32-bit tile offsets
        assert call(ws=100, ex=ex) == api.BASE_ERR_INVALID_ARG
    # the plain entry point takes plain experts only
    assert call(sub=1) == api.BASE_ERR_UNSUPPORTED
    assert call(sub=65, ex=True) == api.BASE_ERR_INVALID_ARG
    assert call(sub=-1, ex=True) == api.BASE_ERR_INVALID_ARG
    assert call(sub=1, eps=-1.0, ex=True) == api.BASE_ERR_INVALID_ARG
    # blocks need the larger workspace
    assert call(sub=1, ws=ws_plain, ex=True) == api.BASE_ERR_INVALID_ARG


def test_backward_workspace_grows_with_blocks(lib):
    T, E, D, F = 65536, 128, 2048, 8192
    bf = api.BASE_BF16
    ex = lambda op, n: api.base_workspace_bytes_ex(op, T, E, D, F, bf, n)
    plain = api.base_workspace_bytes(api.BASE_OP_LAYER_BWD, T, E, D, F, bf)
    assert ex(api.BASE_OP_LAYER_BWD, 0) == plain
    one, two = ex(api.BASE_OP_LAYER_BWD, 1), ex(api.BASE_OP_LAYER_BWD, 2)
    # each block keeps its input, layer-norm output, Z and act(Z)
    assert two - one >= 2 * T * F * 2 + 2 * T * D * 2
    assert one > plain
    assert ex(api.BASE_OP_LAYER_BWD, 65) == 0 and ex(api.BASE_OP_LAYER_BWD, -1) == 0
    # other ops ignore the block count
    assert ex(api.BASE_OP_LAYER, 3) == api.base_workspace_bytes(api.BASE_OP_LAYER, T, E, D, F, bf)
