"""The C-ABI library on the CPU host: it loads, exports every entry point the
public header declares with the signature the boundary documents, and rejects
bad arguments on the host before any HIP call (no GPU is touched by these
tests).  The argument-check tests take the library as a parameter, so that a
host-only sanitized build runs them too (tests/test_host_sanitized.py)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def declared_macros():
    text = open(HEADER).read()
    return dict((m, int(v, 0)) for m, v in re.findall(r"#define\s+(PKV_\w+)\s+\(?(-?\w+)u?\)?", text)
                if re.fullmatch(r"-?(0x[0-9a-fA-F]+|\d+)", v.rstrip("u")) for v in [v.rstrip("u")])


@pytest.fixture(scope="module")
def lib():
    from paged_kv_input_amd import api

    return api._lib


def test_signatures_match_the_documented_boundary(tmp_path):
    """Every declaration in the header has the signature listed in
    tests/abi_signatures.cpp (static_asserts; g++ -fsyntax-only), which
    includes the departures from the first interface plan: the scatter's row
    bytes and strides, pkv_error_string, void* streams, the slot mapping's
    sliding window, and pkv_step_path."""
    src = os.path.join(ROOT, "tests", "abi_signatures.cpp")
    r = subprocess.run(["g++", "-std=c++17", "-fsyntax-only", f"-I{os.path.join(ROOT, 'include')}",
                        src], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    text = open(src).read()
    checked = set(re.findall(r"PKV_SIG\((pkv_\w+),", text))
    assert checked == set(declared_functions())


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(["pkv_abi_version", "pkv_add_requests", "pkv_advance_state",
                     "pkv_append_blocks", "pkv_blocks_needed", "pkv_compute_slot_mapping",
                     "pkv_error_string",
                     "pkv_gather_kv", "pkv_hash_blocks", "pkv_prefix_clear", "pkv_prefix_evict",
                     "pkv_lookahead_slots", "pkv_prefix_insert", "pkv_prefix_lookup",
                     "pkv_prepare_batch", "pkv_row_pool_acquire", "pkv_row_pool_create",
                     "pkv_row_pool_destroy", "pkv_row_pool_num_free", "pkv_row_pool_release",
                     "pkv_scatter_kv", "pkv_step", "pkv_step_path", "pkv_window_free"])
    for name in names:
        assert hasattr(lib, name), name
    so = os.path.join(ROOT, "paged_kv_input_amd", "libpagedkv.so")
    out = subprocess.run(["nm", "-D", "--defined-only", so], check=True, capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (pkv_\w+)", out))
    assert exported == set(names), exported ^ set(names)


def test_constants_match_binding(lib):
    from paged_kv_input_amd import _abi as api
    import oracle

    m = declared_macros()
    assert lib.pkv_abi_version() == m["PKV_ABI_VERSION"]
    assert api.MAX_BATCH == m["PKV_MAX_BATCH"]
    assert api.STEP_MAX_BATCH == m["PKV_STEP_MAX_BATCH"]
    assert api.STEP_MAX_GROUPS == m["PKV_STEP_MAX_GROUPS"]
    assert api.STEP_RANKED_MIN_BATCH == m["PKV_STEP_RANKED_MIN_BATCH"]
    assert ctypes.sizeof(api.Group) == 104
    for name, bit in api.ST_BITS.items():
        assert m["PKV_ST_" + name] == bit
        assert getattr(oracle, "ST_" + name) == bit
    for code in ("OK", "EINVAL", "EALIGN", "EUNSUPPORTED", "EHIP", "ENOROWS", "ENOMEM"):
        assert m["PKV_" + code] == getattr(api, code)
    assert m["PKV_ENOROWS"] == oracle.ENOROWS
    assert (m["PKV_STEP_ONE_LAUNCH"], m["PKV_STEP_BATCH_THEN_SCATTER"], m["PKV_STEP_SEPARATE"],
            m["PKV_STEP_RANKED_ONE_LAUNCH"]) \
        == (api.STEP_ONE_LAUNCH, api.STEP_BATCH_THEN_SCATTER, api.STEP_SEPARATE,
            api.STEP_RANKED_ONE_LAUNCH)
    for code in (0, -1, -2, -3, -4, -5, -6, 99):
        assert api.error_string(lib, code)


def test_host_argument_errors(lib):
    """Each of these returns before anything is enqueued (no HIP call)."""
    N = None
    P = ctypes.c_void_p
    fake = P(0x1000)          # never dereferenced: validation fails first
    EINVAL, EALIGN, EUNSUP = -1, -2, -3
    prep = lib.pkv_prepare_batch
    assert prep(-1, 0, fake, fake, fake, 1, fake, 1, 1, fake, fake, fake, fake, fake, N, N) == EINVAL
    assert prep(1, -1, fake, fake, fake, 1, fake, 1, 1, fake, fake, fake, fake, fake, N, N) == EINVAL
    assert prep(1, 1, fake, fake, fake, 1, fake, 1, 1, fake, N, fake, fake, fake, N, N) == EINVAL
    assert prep(1, 1, N, fake, fake, 1, fake, 1, 1, fake, fake, fake, fake, fake, N, N) == EINVAL
    assert prep(1, 1, fake, fake, fake, 1, fake, 1, 1, fake, fake, fake, N, fake, N, N) == EINVAL
    assert prep(1, 1, fake, fake, fake, 1, fake, 3, 4, fake, fake, fake, fake, fake, N, N) == EINVAL
    assert prep(4097, 1, fake, fake, fake, 1, fake, 1, 1, fake, fake, fake, fake, fake, N, N) == EUNSUP
    slots = lib.pkv_compute_slot_mapping
    assert slots(1, 1, fake, fake, fake, fake, fake, 1, 1, 0, 4, 0, fake, N, N, N) == EINVAL
    assert slots(1, 1, fake, fake, fake, fake, fake, 1, 1, 16, -1, 0, fake, N, N, N) == EINVAL
    assert slots(1, 1, fake, fake, fake, fake, fake, 1, 1, 16, 4, -1, fake, N, N, N) == EINVAL
    assert slots(1, 1, fake, fake, fake, fake, fake, 1, 1, 1 << 16, 1 << 16, 0, fake, N, N, N) == EINVAL
    assert slots(1, 1, fake, fake, N, fake, fake, 1, 1, 16, 4, 0, fake, fake, N, N) == EINVAL
    assert slots(1, 1, fake, fake, fake, fake, fake, 1, 1, 16, 4, 0, N, N, N, N) == EINVAL
    assert slots(4097, 1, fake, fake, fake, fake, fake, 1, 1, 16, 4, 0, fake, N, N, N) == EUNSUP
    sc = lib.pkv_scatter_kv
    assert sc(-1, 16, fake, 16, fake, 16, fake, fake, 4, fake, N, N) == EINVAL
    assert sc(1, 16, fake, 8, fake, 16, fake, fake, 4, fake, N, N) == EINVAL
    assert sc(1, 16, N, 16, fake, 16, fake, fake, 4, fake, N, N) == EINVAL
    assert sc(1, 24, fake, 32, fake, 32, fake, fake, 4, fake, N, N) == EALIGN
    assert sc(1, 16, P(0x1008), 16, fake, 16, fake, fake, 4, fake, N, N) == EALIGN
    assert sc(1, 16, fake, 24, fake, 16, fake, fake, 4, fake, N, N) == EALIGN
    assert sc(1, 16, fake, 16, fake, 16, fake, P(0x1004), 4, fake, N, N) == EALIGN


def test_step_host_argument_errors(lib):
    from paged_kv_input_amd import _abi as api

    P = ctypes.c_void_p
    fake = 0x1000
    g = api.Group(fake, fake, None, fake, fake, fake, fake, 16, 16, 4, 16, 2, 16, 4, 0)
    arr = (api.Group * 1)(g)
    st = lib.pkv_step
    args = [1, 1, fake, fake, fake, 1, fake, 1, 1, fake, fake, fake, fake, fake]
    assert st(*args, -1, arr, None, None) == -1          # num_groups < 0
    assert st(*args, 1, None, None, None) == -1          # groups NULL
    arr[0].sliding_window = -1
    assert st(*args, 1, arr, None, None) == -1           # negative window
    arr[0].sliding_window = 0
    arr[0].block_size = 0
    assert st(*args, 1, arr, None, None) == -1           # group's block size
    arr[0].block_size = 16
    arr[0].row_bytes = 24
    arr[0].k_stride = arr[0].v_stride = 32
    assert st(*args, 1, arr, None, None) == -2           # row not a multiple of 16 bytes
    args[0] = 4097
    arr[0].row_bytes = 16
    assert st(*args, 1, arr, None, None) == -3           # beyond PKV_MAX_BATCH


def test_gather_host_argument_errors(lib):
    N = None
    P = ctypes.c_void_p
    fake = P(0x1000)
    g = lib.pkv_gather_kv
    # n, seq_lens, qsl, window, pages, MB, bs, NB, row_bytes, kc, vc, out_tokens, k_out,
    # k_stride, v_out, v_stride, kv_start, status, stream
    ok = [2, fake, fake, 0, fake, 4, 16, 8, 256, fake, fake, 64, fake, 256, fake, 256, N, N, N]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)

    assert call(a0=-1) == -1                       # n < 0
    assert call(a6=0) == -1                        # block_size <= 0
    assert call(a8=0) == -1                        # row_bytes <= 0
    assert call(a11=-1) == -1                      # out_tokens < 0
    assert call(a13=128) == -1                     # k_out stride < row_bytes
    assert call(a7=1 << 27, a6=32) == -1           # num_blocks * block_size > 2^31
    assert call(a3=-1) == -1                       # negative window
    assert call(a3=8, a2=N) == -1                  # a window needs query_start_loc
    assert call(a1=N) == -1                        # seq_lens NULL
    assert call(a4=N) == -1                        # pages NULL with MB > 0
    assert call(a12=N) == -1                       # k_out NULL
    assert call(a9=N) == -1                        # cache NULL
    assert call(a8=24, a13=32, a15=32) == -2       # row not a multiple of 16
    assert call(a12=P(0x1008)) == -2               # misaligned output
    assert call(a0=4097) == -3                     # beyond PKV_MAX_BATCH
    assert call(a11=1 << 31) == -3                 # out_tokens > INT32_MAX
    assert call(a0=0, a1=N, a4=N, a16=N) == 0      # nothing to do: nothing enqueued


def test_prefix_host_argument_errors(lib):
    N = None
    fake = ctypes.c_void_p(0x1000)
    h = lib.pkv_hash_blocks
    assert h(-1, fake, 8, fake, fake, 4, 2, fake, N, N, N) == -1       # m < 0
    assert h(1, fake, 8, fake, fake, 0, 2, fake, N, N, N) == -1        # block_size <= 0
    assert h(1, fake, -1, fake, fake, 4, 2, fake, N, N, N) == -1       # total < 0
    assert h(1, N, 8, fake, fake, 4, 2, fake, N, N, N) == -1           # tokens NULL
    assert h(1, fake, 8, fake, fake, 4, 2, N, N, N, N) == -1           # hashes NULL
    assert h(0, N, 0, N, N, 4, 2, N, N, N, N) == 0                     # nothing to do
    assert lib.pkv_prefix_clear(fake, fake, 12, N) == -1               # not a power of two
    assert lib.pkv_prefix_clear(N, fake, 16, N) == -1
    assert lib.pkv_prefix_clear(N, N, 0, N) == 0
    lk = lib.pkv_prefix_lookup
    assert lk(1, fake, 2, fake, 4, fake, fake, 6, N, fake, N, N) == -1  # capacity 6
    assert lk(1, fake, 2, fake, 4, fake, fake, 8, N, N, N, N) == -1     # num_computed NULL
    assert lk(1, fake, 2, fake, 0, fake, fake, 8, N, fake, N, N) == -1  # block_size 0
    ins = lib.pkv_prefix_insert
    assert ins(1, fake, 2, fake, fake, fake, fake, 4, fake, fake, -8, N, N) == -1
    assert ins(1, fake, 2, N, fake, fake, fake, 4, fake, fake, 8, N, N) == -1
    assert ins(1, fake, 2, fake, fake, fake, N, 4, fake, fake, 8, N, N) == -1
    ev = lib.pkv_prefix_evict
    assert ev(-1, fake, fake, fake, fake, 8, N) == -1
    assert ev(1, N, fake, fake, fake, 8, N) == -1
    assert ev(0, N, N, N, N, 8, N) == 0


def test_alloc_host_argument_errors(lib):
    N = None
    fake = ctypes.c_void_p(0x1000)
    wf = lib.pkv_window_free
    assert wf(-1, fake, fake, fake, 4, 4, 16, 8, fake, fake, N, N) == -1
    assert wf(1, fake, fake, fake, 4, 4, 0, 8, fake, fake, N, N) == -1      # block_size 0
    assert wf(1, fake, fake, fake, 4, 4, 16, -1, fake, fake, N, N) == -1    # window < 0
    assert wf(1, fake, fake, fake, 4, 4, 16, 8, N, fake, N, N) == -1        # freed NULL
    assert wf(1, fake, fake, N, 4, 4, 16, 8, fake, fake, N, N) == -1        # table NULL
    assert wf(0, N, N, N, 4, 4, 16, 8, N, N, N, N) == 0
    la = lib.pkv_lookahead_slots
    assert la(1, fake, fake, fake, 4, 4, 16, 8, -1, fake, N, N) == -1       # k < 0
    assert la(1, fake, fake, fake, 4, 4, 16, 8, 2, N, N, N) == -1           # out NULL
    assert la(1, fake, fake, fake, 4, 4, 1 << 16, 1 << 16, 2, fake, N, N) == -1
    assert la(3, N, N, N, 4, 4, 16, 8, 0, N, N, N) == 0                      # k = 0
    bn = lib.pkv_blocks_needed
    assert bn(1, fake, fake, -1, 16, fake, fake, 4, fake, N, N) == -1      # k < 0
    assert bn(1, fake, fake, 0, 0, fake, fake, 4, fake, N, N) == -1        # block_size 0
    assert bn(1, fake, fake, 0, 16, fake, fake, 4, N, N, N) == -1          # need NULL
    assert bn(0, N, N, 0, 16, N, N, 4, N, N, N) == 0


def test_state_host_argument_errors(lib):
    """The state updates reject what the oracle rejects, before any HIP call."""
    N = None
    fake = ctypes.c_void_p(0x1000)
    add = lib.pkv_add_requests
    ok = [1, fake, fake, fake, fake, 4, fake, fake, 2, 8, fake, fake, 16, 16, fake, 4, fake, N, N]

    def with_(args, **kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return a

    assert add(*with_(ok, a0=-1)) == -1                 # m < 0
    assert add(*with_(ok, a5=-1)) == -1                 # num_prompt_tokens < 0
    assert add(*with_(ok, a8=-1)) == -1                 # num_blocks_given < 0
    assert add(*with_(ok, a12=8)) == -1                 # token_stride < L
    assert add(*with_(ok, a15=-1)) == -1                # MB < 0
    assert add(*with_(ok, a1=N)) == -1                  # rows NULL
    assert add(*with_(ok, a4=N)) == -1                  # prompt tokens NULL, some given
    assert add(*with_(ok, a7=N)) == -1                  # blocks NULL, some given
    assert add(*with_(ok, a14=N)) == -1                 # block table NULL
    assert add(*with_(ok, a0=0, a1=N, a2=N, a3=N, a6=N)) == 0   # m = 0: nothing to do
    app = lib.pkv_append_blocks
    ok = [1, fake, fake, fake, 2, 8, fake, 4, fake, N, N]
    assert app(*with_(ok, a0=-1)) == -1
    assert app(*with_(ok, a4=-1)) == -1
    assert app(*with_(ok, a7=-1)) == -1
    assert app(*with_(ok, a2=N)) == -1
    assert app(*with_(ok, a8=N)) == -1
    assert app(*with_(ok, a0=0, a1=N, a2=N)) == 0
    adv = lib.pkv_advance_state
    ok = [1, fake, fake, fake, 8, fake, fake, 16, 16, N, N]
    assert adv(*with_(ok, a0=-1)) == -1
    assert adv(*with_(ok, a7=8)) == -1                  # token_stride < L
    assert adv(*with_(ok, a1=N)) == -1
    assert adv(*with_(ok, a6=N)) == -1                  # sampled without a token table
    assert adv(*with_(ok, a0=0, a1=N, a2=N)) == 0


def test_step_path_argument_errors(lib):
    from paged_kv_input_amd import _abi as api

    g = (api.Group * 1)(api.Group(row_bytes=2048, k_stride=2048, v_stride=2048))
    assert lib.pkv_step_path(-1, 0, 1, g) == -1
    assert lib.pkv_step_path(1, -1, 1, g) == -1
    assert lib.pkv_step_path(1, 1, -1, g) == -1
    assert lib.pkv_step_path(1, 1, 1, None) == -1
    assert lib.pkv_step_path(0, 0, 0, None) == api.STEP_BATCH_THEN_SCATTER


def test_binding_rejects_cpu_tensors():
    import torch
    import paged_kv_input_amd as pkv

    x = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError):
        pkv.compute_slot_mapping(x, torch.zeros(4, dtype=torch.int32), x, x,
                                 torch.zeros(2, 2, dtype=torch.int32), 16, 4, slot_mapping=x)
