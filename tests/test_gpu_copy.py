"""GPU checkpoint write / restore: batched page copies, bit-exact, touching only
the state bytes of the destination pages (poisoned pool)."""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
from kda_gpu_util import PoolBuf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,D,page_bytes,npairs", [
    (32, 128, 2 << 20, 256),            # 256 x 2 MiB pages each way
    (32, 128, (2 << 20) + 4096, 37),    # padded pages: padding never touched
    (3, 64, 3 * 64 * 64 * 4, 500),      # more pairs than one launch carries
])
def test_write_then_restore(H, D, page_bytes, npairs):
    pb = PoolBuf(3 * npairs, H, D, page_bytes=page_bytes)
    rng = np.random.default_rng(npairs)
    active = rng.permutation(npairs)
    ckpt = npairs + rng.permutation(npairs)
    restored = 2 * npairs + rng.permutation(npairs)
    # fill the active pages' state bytes with random words
    w = page_bytes // 4
    sw = H * D * D
    for p in active:
        pb.buf[p * w:p * w + sw] = torch.from_numpy(rng.integers(-2**31, 2**31, sw, dtype=np.int64)
                                                    .astype(np.int32)).cuda()
    before = pb.snapshot()
    K.kda_checkpoint_write(pb.pool, active, ckpt)
    K.kda_checkpoint_restore(pb.pool, ckpt, restored)
    torch.cuda.synchronize()
    after = pb.snapshot()
    expect = before.copy()
    for a, c, r in zip(active, ckpt, restored):
        expect[c * w:c * w + sw] = before[a * w:a * w + sw]
        expect[r * w:r * w + sw] = before[a * w:a * w + sw]
    assert np.array_equal(after, expect)


def test_restore_leaves_checkpoint_untouched_under_reuse():
    """Copy-on-write: restoring one checkpoint into several active pages and
    then overwriting those pages never changes the checkpoint."""
    pb = PoolBuf(6, 2, 64)
    pb.buf[:2 * 64 * 64] = torch.arange(2 * 64 * 64, dtype=torch.int32, device="cuda")
    K.kda_checkpoint_write(pb.pool, [0], [1])
    snap = pb.page_words(1).clone()
    K.kda_checkpoint_restore(pb.pool, [1], [2])
    K.kda_checkpoint_restore(pb.pool, [1], [3])
    pb.page_words(2).fill_(7)
    torch.cuda.synchronize()
    assert torch.equal(pb.page_words(1), snap)
    assert torch.equal(pb.page_words(3)[:2 * 64 * 64], pb.page_words(0)[:2 * 64 * 64])
