"""The decode entry point that allocates nothing (sparse_mla_decode_noalloc) against the
workspace entry point (sparse_mla_decode): same kernels and split plan, so the results must be
bitwise equal.  Two calls in a row, the second smaller, both with split-K so the scratch array
carries the partials and (max, sum) pairs; a plan that needs more scratch than the library holds
is refused before anything is launched."""
import pytest
import torch

import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import dev, q_dev, require_gpu
from workload import make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pair(w, splits, out_dtype):
    q, cache = q_dev(w), w.cache.to_device("cuda")
    from sparse_mla_decode_topk_amd.pipeline import DcpDecodeStep
    step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=1, block_size=w.block_size, softmax_scale=w.sm_scale)
    step.run(q, dev(w.ids), dev(w.req), [(cache, dev(w.block_table))])
    slots, valid = step.slots[0], step.valid[0]
    ref_o, ref_l = smla.decode(q, cache, slots, w.sm_scale, out_dtype=out_dtype, num_splits=splits, valid_count=valid)
    out = torch.full_like(ref_o, 7.0)
    lse = torch.full_like(ref_l, 3.0)
    smla.decode_noalloc(q, cache, slots, w.sm_scale, out, lse, num_splits=splits, valid_count=valid)
    torch.cuda.synchronize()
    return ref_o, ref_l, out, lse


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(make_random(71, T=24, H=128, K=640, ctx=4096, B=64, D=1, neg_frac=0.2, n_req=4), 4, torch.float32),
             (make_random(72, T=5, H=64, K=200, ctx=700, B=32, D=1, neg_frac=0.3, n_req=2), 3, torch.bfloat16)]
    for i, (w, splits, od) in enumerate(cases):
        print(f"call {i}: T={w.T} H={w.H} K={w.K} splits={splits} {od}", flush=True)
        ref_o, ref_l, out, lse = _pair(w, splits, od)
        assert torch.equal(out, ref_o), f"call {i}: out differs"
        assert torch.equal(lse, ref_l), f"call {i}: lse differs"


def test_noalloc_refuses_plans_beyond_the_scratch():
    # T=1024 rows, H=128, 8 splits: 1024 * 8 * 128 * 512 * 4 bytes of partials, far above 32 MiB
    T, H, K = 1024, 128, 2048
    q = torch.zeros((T, H, 576), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((64, 656), dtype=torch.uint8, device="cuda")
    slots = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    with pytest.raises(smla.SmlaError) as e:
        smla.decode_noalloc(q, cache, slots, 0.1, out, lse, num_splits=8)
    assert e.value.status == 3  # SMLA_ERR_WORKSPACE
