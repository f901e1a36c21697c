"""Host-side tests of the C ABI (no GPU needed: every call here fails validation
before any HIP call, or is a pure host query)."""
import ctypes
import os
import re
import subprocess

import pytest

import shared_base_residual_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built")

OK, E_NULL, E_SHAPE, E_UNSUP, E_WS, E_ALIGN = 0, -1, -2, -3, -4, -5
FAKE = 0x10000  # never dereferenced: validation fails before any device call


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|void|const char \*)\s*(rattn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    decl = declared_functions()
    assert len(decl) >= 8, decl
    lib = R.lib()
    for name in decl:
        assert hasattr(lib, name), f"{name} declared in rattn.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH], capture_output=True, text=True).stdout
    for name in decl:
        assert re.search(rf"\sT\s{name}$", out, re.M), name
    assert set(decl) == set(R.EXPORTS)


def test_version_and_strings():
    assert R.lib().rattn_version() == 2
    assert R.lib().rattn_status_str(0) == b"ok"
    assert R.lib().rattn_status_str(-4).startswith(b"workspace")
    assert R.lib().rattn_last_hip_error() == 0


def cfg1_desc(**kw):
    base = dict(n_agents=4, n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, q_len=1, prefix_len=32768)
    base.update(kw)
    raw_shared = base.pop("shared_lr", 0)
    d = R.make_desc(**base)
    d.shared_lr = raw_shared  # raw value, so that invalid ones reach the library
    return d


def ws(desc, op=0):
    n = ctypes.c_size_t(0)
    st = R.lib().rattn_workspace_bytes(ctypes.byref(desc), op, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(n_agents=0), E_SHAPE),
    (dict(n_q_heads=30), E_SHAPE),
    (dict(head_dim=96), E_UNSUP),
    (dict(rank=12), E_UNSUP),
    (dict(rank=-1), E_SHAPE),
    (dict(page_size=8, n_phys_pages=4), E_UNSUP),
    (dict(page_size=16, n_phys_pages=0), E_SHAPE),
    (dict(prefix_len=0, priv_len=0), E_SHAPE),
    (dict(prefix_len=-5), E_SHAPE),
    (dict(dtype=7), E_UNSUP),
    (dict(shared_lr=2), E_SHAPE),
    (dict(q_len=0), E_SHAPE),
])
def test_descriptor_validation(kw, status):
    st, _ = ws(cfg1_desc(**kw))
    assert st == status


def test_prefill_requires_chunk_shape():
    d = cfg1_desc(q_len=4, priv_len=3)
    assert ws(d, op=1)[0] == E_SHAPE
    assert ws(cfg1_desc(q_len=3, priv_len=3), op=1)[0] == OK
    assert ws(d, op=5)[0] == E_SHAPE


def test_workspace_null_out_pointer():
    d = cfg1_desc()
    assert R.lib().rattn_workspace_bytes(ctypes.byref(d), 0, None) == E_NULL
    assert R.lib().rattn_workspace_bytes(None, 0, ctypes.byref(ctypes.c_size_t())) == E_NULL


def test_workspace_monotone():
    prev = 0
    for L in (1, 100, 1000, 32768, 100000):
        st, n = ws(cfg1_desc(prefix_len=L))
        assert st == OK and n >= prev
        prev = n
    prev = 0
    for N in (1, 2, 4, 8, 16):
        st, n = ws(cfg1_desc(n_agents=N))
        assert st == OK and n >= prev
        prev = n


def plan(desc):
    return R.decode_plan(desc)


@pytest.mark.parametrize("kw", [
    dict(), dict(prefix_len=8192, priv_len=512, page_size=16, n_phys_pages=1024, n_agents=16, rank=64),
    dict(n_agents=8, n_q_heads=64, prefix_len=65536), dict(n_agents=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                                          rank=8, prefix_len=256, dtype=0),
    dict(prefix_len=1000, priv_len=77), dict(prefix_len=0, priv_len=300), dict(q_len=5),
    dict(n_q_heads=8, n_kv_heads=8, rank=128), dict(shared_lr=1, rank=128, n_agents=32),
])
def test_plan_covers_context(kw):
    d = cfg1_desc(**kw)
    p = plan(d)
    L, S = d.prefix_len, d.priv_len
    if L:
        assert p["prefix_split_len"] % 128 == 0
        assert p["n_prefix_splits"] * p["prefix_split_len"] >= L
        assert p["prefix_split_len"] - 128 < -(-L // p["n_prefix_splits"])
    else:
        assert p["n_prefix_splits"] == 0
    if S:
        assert p["priv_split_len"] % 128 == 0
        assert p["n_priv_splits"] * p["priv_split_len"] >= S
        assert p["priv_split_len"] - 128 < -(-S // p["n_priv_splits"])
    g = d.n_q_heads // d.n_kv_heads
    rpa = d.q_len * g
    if rpa <= 16:
        assert p["agents_per_block"] * rpa <= 16
        if d.rank and not d.shared_lr and L:
            if p["masked"]:  # U and W are the rank wide, several agents per block
                assert d.dtype == 1 and d.rank >= 32 and p["resid_cols"] == d.rank and p["agents_per_block"] > 1
            else:
                assert p["agents_per_block"] * d.rank <= p["resid_cols"] <= 128
        assert p["row_blocks"] * p["agents_per_block"] >= d.n_agents
    if d.rank and L:
        assert p["resid_cols"] in (32, 64, 128)
    rg = -(-p["row_blocks"] // p["blocks_per_group"])
    pb = 1 if rpa <= 16 else -(-rpa // 16)
    H = p["heads_per_item"]
    assert H >= 1 and d.n_kv_heads % H == 0 and (H == 1 or (d.rank and L))
    items = (p["n_prefix_splits"] * rg * (d.n_kv_heads // H)
             + d.n_agents * (-(-pb // 4)) * p["n_priv_splits"] * d.n_kv_heads)
    assert p["work_items"] == items


def args(**kw):
    a = dict(q=FAKE, k_base=FAKE, v_base=FAKE, block_table=None, lk=FAKE, lv=FAKE, bk=FAKE, bv=FAKE,
             k_priv=None, v_priv=None, out=FAKE, lse=None)
    a.update(kw)
    return R.Args(*[a.get(n) for n, _ in R.Args._fields_])


def call(desc, a, ws_ptr=FAKE, ws_bytes=1 << 40, fn="rattn_decode"):
    return getattr(R.lib(), fn)(ctypes.byref(desc), ctypes.byref(a), ctypes.c_void_p(ws_ptr),
                                ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_NULL),
    (dict(out=None), E_NULL),
    (dict(k_base=None), E_NULL),
    (dict(lk=None), E_NULL),
    (dict(bv=None), E_NULL),
    (dict(block_table=FAKE), E_NULL),        # table given for a contiguous cache
    (dict(q=FAKE + 8), E_ALIGN),
    (dict(lv=FAKE + 2), E_ALIGN),
    (dict(lse=FAKE + 2), E_ALIGN),
])
def test_argument_validation(kw, status):
    assert call(cfg1_desc(), args(**kw)) == status


def test_private_tokens_need_pointers():
    d = cfg1_desc(priv_len=64)
    assert call(d, args()) == E_NULL
    assert call(d, args(k_priv=FAKE)) == E_NULL


def test_paged_needs_table():
    d = cfg1_desc(page_size=16, n_phys_pages=4096)
    assert call(d, args()) == E_NULL


def test_workspace_checks():
    d = cfg1_desc()
    _, need = ws(d)
    assert need > 0
    assert call(d, args(), ws_ptr=0, ws_bytes=need) == E_WS
    assert call(d, args(), ws_ptr=FAKE, ws_bytes=need - 1) == E_WS
    assert call(d, args(), ws_ptr=FAKE + 16, ws_bytes=need) == E_ALIGN


def test_invalid_descriptor_before_arguments():
    assert call(cfg1_desc(head_dim=80), args(q=None)) == E_UNSUP
    assert R.lib().rattn_decode(None, None, None, 0, None) == E_NULL
    assert call(cfg1_desc(), args(), fn="rattn_prefill_chunk") == E_SHAPE  # q_len != priv_len


def test_gather_validation():
    L = R.lib()
    d = cfg1_desc(page_size=16, n_phys_pages=8, prefix_len=100)
    assert L.rattn_gather_base(ctypes.byref(d), None, FAKE, FAKE, None) == E_NULL
    assert L.rattn_gather_base(ctypes.byref(d), FAKE + 4, FAKE, FAKE, None) == E_ALIGN
    assert L.rattn_gather_base(ctypes.byref(cfg1_desc(page_size=0)), FAKE, FAKE, FAKE, None) == E_UNSUP
    assert L.rattn_gather_base(ctypes.byref(cfg1_desc(page_size=16, n_phys_pages=0)), FAKE, FAKE, FAKE,
                               None) == E_SHAPE
    assert L.rattn_gather_base(ctypes.byref(cfg1_desc(page_size=16, n_phys_pages=4, prefix_len=0)), None,
                               None, None, None) == OK


def test_check_block_table_validation():
    """rattn_check_block_table: every check before any HIP call."""
    L = R.lib()
    f = L.rattn_check_block_table
    d = cfg1_desc(page_size=16, n_phys_pages=8, prefix_len=100)
    assert f(ctypes.byref(d), FAKE, None, None) == E_NULL
    assert f(None, FAKE, FAKE, None) == E_NULL
    assert f(ctypes.byref(d), None, FAKE, None) == E_NULL
    assert f(ctypes.byref(d), FAKE + 2, FAKE, None) == E_ALIGN
    assert f(ctypes.byref(d), FAKE, FAKE + 1, None) == E_ALIGN
    assert f(ctypes.byref(cfg1_desc(page_size=0)), FAKE, FAKE, None) == E_UNSUP
    assert f(ctypes.byref(cfg1_desc(page_size=24, n_phys_pages=8)), FAKE, FAKE, None) == E_UNSUP
    assert f(ctypes.byref(cfg1_desc(page_size=16, n_phys_pages=-1)), FAKE, FAKE, None) == E_SHAPE


def test_stage_mask_validation():
    """rattn_attention_stages accepts only a non-empty subset of split | combine,
    and only the two ops; all checked before any HIP call."""
    L = R.lib()
    d = cfg1_desc()
    _, need = ws(d)
    a = args()
    for stages in (0, 4, 7):
        assert L.rattn_attention_stages(ctypes.byref(d), 0, ctypes.byref(a), FAKE, need, None, stages) == E_SHAPE
    assert L.rattn_attention_stages(ctypes.byref(d), 5, ctypes.byref(a), FAKE, need, None, 1) == E_SHAPE
    assert L.rattn_attention_stages(ctypes.byref(d), 0, ctypes.byref(a), FAKE, need - 1, None, 1) == E_WS


def test_row_limit_and_output_index():
    """The merge writes out[row * d + column] with a 64-bit index; the row
    count a call may have is bounded at 2^28 (d = 128 gives 2^35 elements)."""
    assert ws(cfg1_desc(n_agents=2 ** 21, n_q_heads=256, n_kv_heads=8, prefix_len=16))[0] == E_UNSUP
    st, n = ws(cfg1_desc(n_agents=2 ** 15, n_q_heads=128, n_kv_heads=8, prefix_len=16, rank=0))
    assert st == OK and n > 0  # 2^22 rows: planned, index well inside 64 bits


def test_workspace_cache_key_is_the_launch_stream():
    """Calls launched on different streams never share a cached workspace (the
    key is the stream the call is launched on, not the current stream)."""
    class S:
        def __init__(self, h):
            self.cuda_stream = h

    assert R._ws_key("cuda:0", S(1)) != R._ws_key("cuda:0", S(2))
    assert R._ws_key("cuda:0", S(1)) == R._ws_key("cuda:0", S(1))
    assert R._ws_key("cuda:0", S(1)) != R._ws_key("cuda:1", S(1))
