"""Host checks that tests/kernel_paths.py reaches every kernel instantiation.

The planner (host code in librattn, no GPU needed) decides which kernel a call
runs; these tests pin that each listed workload lands on its instantiation and
that the list covers all of them, so the GPU parity test over the list runs
every kernel the library can launch."""
import os

import pytest

import shared_base_residual_amd as R
from tests import kernel_paths as KP

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built")


def desc_of(c, k8=False):
    return R.make_desc(n_agents=c.n_agents, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                       rank=c.rank, q_len=c.q_len, prefix_len=c.prefix_len, priv_len=c.priv_len,
                       page_size=c.page_size, shared_lr=c.shared_lr, n_phys_pages=c.n_phys_pages,
                       dtype=R.RATTN_BF16 if c.dtype == "bf16" else R.RATTN_F32,
                       k_format=R.RATTN_KEYS_INT8 if k8 else R.RATTN_KEYS_DTYPE, k_scale=0.03 if k8 else 0.0)


def op_of(c):
    return R.RATTN_OP_PREFILL if c.mode == "prefill" else R.RATTN_OP_DECODE


@pytest.mark.parametrize("key,case", KP.PATHS, ids=[c.name for _, c in KP.PATHS])
def test_workload_reaches_its_kernel(key, case):
    assert R.kernel_of(desc_of(case), op_of(case)) == key


@pytest.mark.parametrize("key,case", KP.PATHS_K8, ids=[c.name for _, c in KP.PATHS_K8])
def test_int8_key_workload_reaches_its_kernel(key, case):
    assert R.kernel_of(desc_of(case, k8=True), R.RATTN_OP_DECODE) == key


def test_every_built_kernel_is_listed():
    listed = {k for k, _ in KP.PATHS} | {k for k, _ in KP.PATHS_K8}
    assert listed == KP.built_instantiations()


def test_fp32_widest_residual_unsupported():
    """fp32 at d = 128 with 128 residual columns has no instantiation (its
    registers would spill): decode and prefill both refuse it."""
    from tests.kernel_paths import _dec, _pre

    for c in (_dec(1, 2, 2, 128, 128, 500, dtype="f32"), _pre(1, 2, 2, 128, 128, 500, 20, dtype="f32")):
        with pytest.raises(R.RattnError) as e:
            R.plan(desc_of(c), op_of(c))
        assert e.value.status == -3
