"""pkv_step's launch plan on the CPU: pkv_step_path's value at the edges of
each rule (batch size, tokens per request, group count, 32-bit tile
offsets), and -- through a host-only build whose launchers only log (see
host_lib.py) -- the launches pkv_step really enqueues for the same arguments.
Both paths give the same results (the GPU tests compare them); these tests pin
which one runs.  The checks take the library as a parameter, so the sanitized
host build runs them too."""
import ctypes
import os

import pytest

from paged_kv_input_amd import _abi

HERE = os.path.dirname(os.path.abspath(__file__))
FAKE = 0x1000           # never dereferenced: the stub launchers enqueue nothing


def groups(num, row_bytes=2048, k_stride=None, v_stride=None, pages=True):
    arr = (_abi.Group * max(num, 1))()
    for i in range(num):
        arr[i] = _abi.Group(FAKE, FAKE, FAKE if pages else None, FAKE, FAKE, FAKE, FAKE,
                            k_stride or row_bytes, v_stride or row_bytes, 1 << 20, row_bytes,
                            64, 16, 1 << 16, 0)
    return arr


# (n, T, num_groups, group kwargs, expected plan).  The rules, restated:
# with 1..4 groups, n >= 32 and T <= 8 n (T <= 16 n past 256 requests): the
# request-ranked single launch; otherwise the tile launch for n <= 512, unless
# a tile's rows span more than 2^32 16-byte chunks of K or V; otherwise the
# batch with slots and pages then the scatters for <= 4 groups, else the
# separate kernels.
ONE, BATCH, SEP, RANKED = (_abi.STEP_ONE_LAUNCH, _abi.STEP_BATCH_THEN_SCATTER,
                           _abi.STEP_SEPARATE, _abi.STEP_RANKED_ONE_LAUNCH)
# 2 KiB rows: 8-token tiles, 7 rows past the first; 16 B rows: 256-token tiles
S2K = (2**32 - 128) // 7            # largest 16-byte stride that fits with 2 KiB rows
S16 = (2**32 - 1) // 255            # and with 16-byte rows
CASES = [
    (31, 31, 1, {}, ONE),                        # 31 decodes: the tile launch
    (32, 32, 1, {}, RANKED),                     # 32 decodes: ranked
    (32, 256, 1, {}, RANKED),                    # T = 8 n
    (32, 257, 1, {}, ONE),                       # T = 8 n + 1
    (256, 2048, 1, {}, RANKED),
    (256, 2049, 1, {}, ONE),                     # 8 n + 1 at 256 requests
    (257, 4112, 1, {}, RANKED),                  # T = 16 n past 256 requests
    (257, 4113, 1, {}, ONE),
    (512, 8192, 1, {}, RANKED),
    (512, 8193, 1, {}, ONE),
    (513, 16 * 513, 1, {}, RANKED),
    (513, 16 * 513 + 1, 1, {}, BATCH),           # past PKV_STEP_MAX_BATCH, longer requests
    (4096, 4096, 2, {}, RANKED),
    (4096, 65536, 4, {}, RANKED),                # 16 tokens each, four groups
    (4096, 65537, 4, {}, BATCH),
    (4096, 4096, 5, {}, SEP),                    # past PKV_STEP_MAX_GROUPS
    (256, 256, 0, {}, BATCH),                    # no group: the batch alone
    (16, 32768, 4, {}, ONE),
    (16, 32768, 5, {}, SEP),
    (16, 32768, 0, {}, BATCH),
    (16, 32768, 1, dict(k_stride=16 * S2K), ONE),
    (16, 32768, 1, dict(k_stride=16 * (S2K + 1)), BATCH),
    (16, 32768, 1, dict(v_stride=16 * (S2K + 1)), BATCH),
    (64, 64, 1, dict(k_stride=16 * (S2K + 1)), RANKED),  # 64-bit offsets in the ranked launch
    (16, 32768, 1, dict(row_bytes=16, k_stride=16 * S16, v_stride=16 * S16), ONE),
    (16, 32768, 1, dict(row_bytes=16, v_stride=16 * (S16 + 1)), BATCH),
    (2, 9, 1, dict(pages=False), ONE),
]


def check_plans(lib):
    for n, T, ng, kw, want in CASES:
        got = lib.pkv_step_path(n, T, ng, groups(ng, **kw))
        assert got == want, (n, T, ng, kw, got, want)


def check_routing(lib):
    """pkv_step enqueues exactly the launches of pkv_step_path's plan."""
    import host_lib

    for n, T, ng, kw, want in CASES:
        arr = groups(ng, **kw)
        f = FAKE
        rc, log = host_lib.launches(lib, lib.pkv_step, n, T, f, f, f, 1024, f, 8192, 8192, f, f,
                                    f, f, f, ng, arr, None, None)
        assert rc == 0, (n, T, ng, kw, rc)
        if want == ONE:
            expect = ["step"]
        elif want == RANKED:
            expect = [f"prepare+{ng}+kv"]
        elif want == BATCH:
            expect = [f"prepare+{ng}"] + ["scatter"] * ng
        else:
            expect = ["prepare+0"] + ["slots"] * ng + ["scatter"] * ng
        assert log == expect, (n, T, ng, kw, log)
        assert lib.pkv_step_path(n, T, ng, arr) == want


@pytest.fixture(scope="module")
def host_build(tmp_path_factory):
    import host_lib

    return host_lib.load(host_lib.build(str(tmp_path_factory.mktemp("host") / "libpkv_host.so")))


def test_plans_of_the_library():
    from paged_kv_input_amd.api import _lib

    check_plans(_lib)


def test_plans_and_routing_of_the_host_build(host_build):
    check_plans(host_build)
    check_routing(host_build)


def test_stub_log_is_the_only_difference(host_build):
    """The host build's entry points return what the library's return for the
    same (host-rejected) arguments: the same source, no GPU."""
    from paged_kv_input_amd.api import _lib

    P = ctypes.c_void_p
    f = P(FAKE)
    for args in [(1, 16, f, 8, f, 16, f, f, 4, f, None, None),
                 (1, 24, f, 32, f, 32, f, f, 4, f, None, None),
                 (-1, 16, f, 16, f, 16, f, f, 4, f, None, None)]:
        assert host_build.pkv_scatter_kv(*args) == _lib.pkv_scatter_kv(*args)
