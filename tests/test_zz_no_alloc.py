"""GPU check of kda_prefill_chunked_noalloc (the prefill on the library's static
device scratch, for callers that cannot allocate): through the C ABI, two calls
in a row, the second smaller than the first, each bit-identical (o, every
checkpoint and final state, untouched pages) to kda_prefill_chunked with a
workspace of its own on the same inputs.  The first call is longer than one
window of the 64 MiB scratch, so it also runs in more windows than the
workspace call."""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
from kda_gpu_util import PoolBuf, inputs_to_dev, workspace

pytestmark = pytest.mark.gpu

H, D = 32, 128


def _case(seed, lens, sp, dtype):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ns = len(lens)
    s_in = [-1] * ns
    s_in[-1] = 2 * ns  # the last sequence resumes from a stored state
    s_out = list(range(ns))
    ck_cu, ck_pos, ck_page = [0], [], []
    for i in range(ns):
        for pos in range((sp[i] // 512 + 1) * 512, sp[i] + lens[i] + 1, 1536):
            ck_pos.append(pos)
            ck_page.append(2 * ns + 1 + len(ck_page))
        ck_cu.append(len(ck_pos))
    d = G.kda_tokens(seed, H, D, 0, int(cu[-1]), dtype)
    return dict(cu=cu, sp=sp, s_in=s_in, s_out=s_out, ck=dict(ckpt_cu=ck_cu, ckpt_pos=ck_pos,
                ckpt_page=ck_page), npages=2 * ns + 1 + len(ck_pos), di=inputs_to_dev(d, dtype))


def _run(c, dtype, noalloc, s0):
    pb = PoolBuf(c["npages"], H, D)
    pb.set_states(len(c["s_in"]) * 2, s0)
    T = int(c["cu"][-1])
    o = torch.full((T, H, D), float("nan"), device="cuda",
                   dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    di = c["di"]
    kw = dict(start_pos=c["sp"], state_in_page=c["s_in"], state_out_page=c["s_out"], **c["ck"])
    if noalloc:
        K.kda_prefill_chunked_noalloc(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o,
                                      c["cu"], **kw)
    else:
        ind = K.KDA_BF16 if dtype == "bf16" else K.KDA_F32
        ws = workspace(pb.pool, T, len(c["s_in"]), len(c["ck"]["ckpt_pos"]), ind)
        K.kda_prefill_chunked(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, c["cu"],
                              workspace=ws, **kw)
    torch.cuda.synchronize()
    bits = o.view(torch.int16) if dtype == "bf16" else o.view(torch.int32)
    return bits.cpu().numpy(), pb.snapshot()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call(dtype):
    s0 = (np.random.default_rng(5).standard_normal((H, D, D)) / np.sqrt(D)).astype(np.float32)
    big = _case(71, [3000, 2200, 1800], [0, 0, 1024], dtype)  # 110 chunks
    small = _case(72, [700], [512], dtype)
    print(f"noalloc {dtype}: calls of {int(big['cu'][-1])} then {int(small['cu'][-1])} tokens",
          flush=True)
    for c in (big, small):
        o_ws, pool_ws = _run(c, dtype, False, s0)
        o_na, pool_na = _run(c, dtype, True, s0)
        assert np.array_equal(o_ws, o_na)
        assert np.array_equal(pool_ws, pool_na)
