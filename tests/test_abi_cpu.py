"""CPU-side checks of the C ABI: the library loads, exports every symbol the header
declares, and its host-side argument checks behave (no GPU work is launched)."""
import ctypes
import os
import re

import pytest

from sampled_softmax_cross_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "sampled_ce.h")).read()
    return sorted(set(re.findall(r"^SCE_API\s+(?:sce_status|const char\*|int)\s+(\w+)\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from sampled_softmax_cross_amd import build
        build.build()
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_the_header():
    src = open(os.path.join(ROOT, "include", "sampled_ce.h")).read()
    define = lambda name: int(re.search(rf"#define\s+{name}\s+\(?(\d+)", src).group(1))
    assert binding.MAX_V_SAMPLED == define("SCE_MAX_V_SAMPLED")
    assert binding.MAX_V == define("SCE_MAX_V")
    assert binding.MAX_D == define("SCE_MAX_D")
    assert binding.DEV_SCALE_RANGE == define("SCE_DEV_SCALE_RANGE")
    enum = re.search(r"typedef enum sce_dtype \{([^}]*)\}", src).group(1)
    codes = {k: int(v) for k, v in re.findall(r"(SCE_\w+)\s*=\s*(\d+)", enum)}
    assert codes == {"SCE_F32": binding.SCE_F32, "SCE_BF16": binding.SCE_BF16,
                     "SCE_E4M3": binding.SCE_E4M3, "SCE_E4M3_BF16W": binding.SCE_E4M3_BF16W}
    assert binding.REFRESH_WORKSPACE_BYTES == define("SCE_REFRESH_WORKSPACE_BYTES")


def test_version_and_status_strings(lib):
    assert lib.sce_abi_version() == 2
    for code in range(4):
        assert lib.sce_status_string(code).decode().startswith("SCE_")
    assert lib.sce_status_string(99) == b"unknown sce_status"


def _ws(T, d, V, P, dt):
    out = ctypes.c_size_t(0)
    rc = binding.load_library().sce_workspace_size(T, d, V, P, dt, ctypes.byref(out))
    return rc, out.value


def test_workspace_size_host_checks(lib):
    rc, n = _ws(16384, 768, 50304, 10240, binding.SCE_BF16)
    assert rc == 0
    # the [T, P] logits buffer dominates
    assert n >= 16384 * 10240 * 2
    rc0, n0 = _ws(49152, 768, 50304, 0, binding.SCE_BF16)
    assert rc0 == 0 and n0 >= 49152 * 50304 * 2
    assert _ws(10, 7, 100, 10, binding.SCE_BF16)[0] == 1      # d not a multiple of 8
    assert _ws(10, 8, 100, 101, binding.SCE_BF16)[0] == 1     # P > V
    assert _ws(10, 8, 100, -1, binding.SCE_BF16)[0] == 1      # P < 0
    assert _ws(10, 8, 100, 10, 7)[0] == 1                     # bad dtype
    assert _ws(-1, 8, 100, 10, 0)[0] == 1                     # T < 0
    assert _ws(10, 8, 131073, 10, 0)[0] == 1                 # V too large for a candidate build
    assert _ws(10, 8, 1 << 20, 0, 0)[0] == 0                  # ... fine for the full softmax
    assert _ws(10, 8, (1 << 20) + 1, 0, 0)[0] == 1            # beyond the full-softmax limit
    assert _ws(1 << 20, 1 << 14, 4096, 64, 1)[0] == 0         # T * d == 2^34 is the largest
    assert _ws((1 << 20) + 1, 1 << 14, 4096, 64, 1)[0] == 1   # T * d beyond 2^34
    assert lib.sce_workspace_size(1, 8, 8, 1, 0, None) == 1   # null output pointer


def test_forward_backward_host_checks(lib):
    f = lib.sampled_ce_forward_backward
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    args = dict(x=fake, W=fake, y=fake, p=None, T=4, d=8, V=16, P=4, stride=3, off=0, dt=0,
                loss=fake, dX=fake, dW=fake, c=None, tp=None, pp=None, lse=None, rl=None,
                aux=None, ws=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call() == 2                                  # no workspace
    assert call(stride=4) == 1                          # gcd(4, 16) != 1
    assert call(P=17) == 1                              # P > V
    assert call(d=12) == 1                              # d % 8 != 0
    assert call(W=None) == 1
    assert call(x=ctypes.c_void_p((1 << 20) + 2)) == 1  # misaligned
    assert call(ws=fake, wsb=16) == 2                   # too small
    b = lib.sce_build_candidates
    assert b(fake, None, 4, 16, 0, 3, 0, fake, None, fake, None, None, fake, 1 << 30, None) == 1  # P = 0
    assert b(fake, None, 4, 16, 4, 2, 0, fake, None, fake, None, None, fake, 1 << 30, None) == 1  # gcd


def test_building_block_host_checks(lib):
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    out = ctypes.c_size_t(0)
    assert lib.sce_ce_rows_workspace_size(100, ctypes.byref(out)) == 0 and out.value >= 100 * 12
    assert lib.sce_ce_rows_workspace_size(-1, ctypes.byref(out)) == 1
    assert lib.sce_ce_rows_workspace_size(4, None) == 1
    ce = dict(Z=fake, ldz=16, T=4, P=10, dt=1, tp=fake, pp=None, loss=fake, rl=None, lse=None,
              aux=None, ws=None, wsb=0, s=None)

    def cer(**kw):
        a = dict(ce, **kw)
        return lib.sce_ce_rows(*a.values())

    assert cer() == 2                           # no workspace
    assert cer(ldz=12) == 1                     # ldz % 8 != 0
    assert cer(ldz=8) == 1                      # ldz < P
    assert cer(P=0) == 1
    assert cer(dt=7) == 1
    assert cer(loss=None) == 1
    assert cer(tp=None) == 1
    assert cer(Z=ctypes.c_void_p((1 << 20) + 4)) == 1  # misaligned
    assert cer(ws=fake, wsb=16) == 2                   # too small
    g = lib.sce_gather_rows
    assert g(fake, 16, 12, fake, 4, 1, fake, 16, None, None) == 1   # d % 8 != 0
    assert g(fake, 16, 16, fake, 4, 1, fake, 8, None, None) == 1    # ld_out < d
    assert g(fake, 16, 16, None, 4, 1, fake, 16, None, None) == 1   # null indices
    assert g(fake, 0, 16, fake, 4, 1, fake, 16, None, None) == 1    # empty table
    assert g(fake, 16, 16, fake, 4, 5, fake, 16, None, None) == 1   # dtype
    assert g(None, 16, 16, None, 0, 1, None, 16, None, None) == 0   # nothing to gather


def test_fp8_host_checks(lib):
    out = ctypes.c_size_t(0)
    assert lib.sce_workspace_size(16384, 768, 50304, 10240, binding.SCE_E4M3, ctypes.byref(out)) == 0
    assert out.value >= 16384 * 10240 * 2 + 16384 * 10240          # bf16 logits + e4m3 gradient
    assert lib.sce_workspace_size(16, 24, 100, 10, binding.SCE_E4M3, ctypes.byref(out)) == 1  # d % 16
    f = lib.sampled_ce_forward_backward_fp8
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    args = dict(x=fake, W8=fake, ws=ctypes.c_float(0.01), wsd=None, y=fake, p=None, T=4, d=16, V=16, P=4,
                stride=3, off=0, loss=fake, dX=fake, dW=fake, c=None, tp=None, pp=None, lse=None,
                rl=None, aux=None, sc=None, wsp=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call() == 2                                   # no workspace
    assert call(ws=ctypes.c_float(0.0)) == 1             # scale must be > 0
    assert call(ws=ctypes.c_float(float("nan"))) == 1
    assert call(ws=ctypes.c_float(float("inf"))) == 1
    assert call(d=8) == 1                                # d % 16 != 0
    assert call(stride=4) == 1                           # gcd(4, 16) != 1
    assert call(W8=None) == 1
    assert call(x=ctypes.c_void_p((1 << 20) + 8)) == 1   # misaligned
    assert call(wsp=fake, wsb=16) == 2                   # too small
    # a device scale replaces the host one (checked on the device), so a bad host value
    # with a device scale passes the host checks (and stops at the workspace)
    assert call(ws=ctypes.c_float(0.0), wsd=fake) == 2
    assert call(ws=ctypes.c_float(0.0), wsd=ctypes.c_void_p((1 << 20) + 2)) == 1  # misaligned
    g = lib.sampled_ce_forward_backward
    assert g(fake, fake, fake, None, 4, 16, 16, 4, 3, 0, binding.SCE_E4M3, fake, fake, fake, None, None,
             None, None, None, None, None, 0, None) == 1  # the e4m3 step has its own entry point



def test_fp8_bf16w_host_checks(lib):
    out = ctypes.c_size_t(0)
    assert lib.sce_workspace_size(16384, 768, 50304, 10240, binding.SCE_E4M3_BF16W, ctypes.byref(out)) == 0
    sampled = out.value
    assert lib.sce_workspace_size(16384, 768, 50304, 10240, binding.SCE_E4M3, ctypes.byref(out)) == 0
    assert sampled == out.value                          # the same plan when P > 0
    assert lib.sce_workspace_size(4096, 768, 50304, 0, binding.SCE_E4M3_BF16W, ctypes.byref(out)) == 0
    full_own = out.value
    assert lib.sce_workspace_size(4096, 768, 50304, 0, binding.SCE_E4M3, ctypes.byref(out)) == 0
    assert full_own >= out.value + 50304 * 768           # P = 0: room for every row's codes
    assert lib.sce_workspace_size(16, 24, 100, 10, binding.SCE_E4M3_BF16W, ctypes.byref(out)) == 1
    f = lib.sampled_ce_forward_backward_fp8_bf16w
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    args = dict(x=fake, W=fake, y=fake, p=None, T=4, d=16, V=16, P=4, stride=3, off=0, loss=fake,
                dX=fake, dW=fake, c=None, tp=None, pp=None, lse=None, rl=None, aux=None, sc=None,
                wsp=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call() == 2                                   # no workspace
    assert call(d=8) == 1                                # d % 16 != 0
    assert call(stride=4) == 1                           # gcd(4, 16) != 1
    assert call(W=None) == 1
    assert call(W=ctypes.c_void_p((1 << 20) + 8)) == 1   # misaligned
    assert call(y=None) == 1                             # T > 0 needs targets
    assert call(wsp=fake, wsb=16) == 2                   # too small
    g = lib.sampled_ce_forward_backward
    assert g(fake, fake, fake, None, 4, 16, 16, 4, 3, 0, binding.SCE_E4M3_BF16W, fake, fake, fake,
             None, None, None, None, None, None, None, 0, None) == 1  # its own entry point


def test_fp8_prebuilt_host_checks(lib):
    f = lib.sampled_ce_forward_backward_fp8_prebuilt
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    args = dict(x=fake, W8=fake, ws=ctypes.c_float(0.01), wsd=None, c=fake, tp=fake, pp=None,
                aux_in=None, T=4, d=16, V=16, P=4, loss=fake, dX=fake, dW=fake, lse=None, rl=None,
                aux=None, sc=None, wsp=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call() == 2                                   # no workspace
    assert call(P=0) == 1                                # a sampled set only
    assert call(c=None) == 1
    assert call(tp=None) == 1                            # T > 0 needs the target positions
    assert call(ws=ctypes.c_float(0.0)) == 1             # host scale must be > 0
    assert call(ws=ctypes.c_float(0.0), wsd=fake) == 2   # a device scale replaces it
    assert call(d=8) == 1                                # d % 16 != 0
    assert call(x=ctypes.c_void_p((1 << 20) + 8)) == 1   # misaligned
    assert call(V=binding.MAX_V_SAMPLED + 1, P=4) == 1   # the sampled path's V limit


def test_refresh_host_checks(lib):
    r = lib.sce_refresh_e4m3_cache
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    nb = binding.REFRESH_WORKSPACE_BYTES
    args = dict(W=fake, V=16, d=16, W8=fake, sc=fake, st=None, wsp=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return r(*a.values())

    assert call() == 2                                    # no workspace
    assert call(wsp=fake, wsb=nb - 1) == 2                # too small
    assert call(wsp=ctypes.c_void_p((1 << 20) + 64), wsb=nb) == 2  # misaligned workspace
    assert call(d=8, wsp=fake, wsb=nb) == 1               # d % 16 != 0
    assert call(V=0, wsp=fake, wsb=nb) == 1
    assert call(V=binding.MAX_V + 1, wsp=fake, wsb=nb) == 1
    assert call(W=None, wsp=fake, wsb=nb) == 1
    assert call(sc=None, wsp=fake, wsb=nb) == 1
    assert call(W8=ctypes.c_void_p((1 << 20) + 8), wsp=fake, wsb=nb) == 1
    assert call(st=ctypes.c_void_p((1 << 20) + 2), wsp=fake, wsb=nb) == 1


def test_noalloc_build_host_checks(lib):
    """The scratch limit and the argument checks of sce_build_candidates_noalloc are
    decided on the host, before the scratch is looked up or anything is enqueued."""
    f = lib.sce_build_candidates_noalloc
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails on the host
    # prefix positions kept in the scratch: 4 bytes per token beyond the fixed pieces
    big_T = (1 << 20) // 4
    assert f(fake, fake, big_T, 50304, 10240, 20011, 0, fake, None, fake, None, None, None) == 2
    assert f(fake, fake, 100, 50304, 0, 20011, 0, fake, None, fake, None, None, None) == 1   # P = 0
    assert f(fake, fake, 100, 50304, 10, 2, 0, fake, None, fake, None, None, None) == 1      # gcd != 1
    assert f(fake, fake, 100, 131073, 10, 1, 0, fake, None, fake, None, None, None) == 1     # V too large
    assert f(fake, None, 100, 500, 10, 7, 0, None, None, fake, None, None, None) == 1        # no C output
