"""GPU parity of kda_short_conv against oracle/conv.py: outputs within the fp32
rounding bound of the fp64 oracle (plus one bf16 rounding for bf16 outputs),
element by element; final and checkpoint windows bit-exact; pages outside the
call untouched; a split call and a resume from a checkpoint window reproduce
the single call bit for bit; the fused q|k|v workload the bench times
(8192 tokens x 12288 channels) at full size."""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
from kda_gpu_util import POISON_WORD, rel_fro
from oracle import conv

pytestmark = pytest.mark.gpu
POISON = np.int32(np.uint32(POISON_WORD).view(np.int32))
U32 = 2.0 ** -24   # fp32 unit roundoff
UBF = 2.0 ** -8    # bf16 unit roundoff (8 significant bits)


def to64(x, dtype):
    """Generator output (bf16 bits or fp32) -> float64 values."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def to_bits(v, dtype):
    """Exactly representable float64 values -> stored words (uint16 bf16 bits / fp32)."""
    if dtype == "bf16":
        f = v.astype(np.float32)
        assert np.array_equal(f.astype(np.float64), v)
        bits = f.view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), "not a bf16 value"
        return (bits >> 16).astype(np.uint16)
    return v.astype(np.float32)


def dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


class ConvPool:
    """A poisoned device region of conv-window pages."""

    def __init__(self, num_pages, C, W, dtype, extra=256):
        self.C, self.W, self.dtype = C, W, dtype
        self.elem = 2 if dtype == "bf16" else 4
        self.win_bytes = (W - 1) * C * self.elem
        self.page_bytes = (self.win_bytes + extra + 255) // 256 * 256
        self.buf = torch.full((num_pages * self.page_bytes // 4,), int(POISON), dtype=torch.int32,
                              device="cuda")
        code = K.KDA_BF16 if dtype == "bf16" else K.KDA_F32
        self.pool = K.make_conv_pool(self.buf, self.page_bytes, num_pages, C, W, code)

    def _bytes(self, p):
        return self.buf.view(torch.uint8)[p * self.page_bytes:(p + 1) * self.page_bytes]

    def set_window(self, p, v64):
        raw = np.ascontiguousarray(to_bits(v64, self.dtype)).view(np.uint8).reshape(-1)
        self._bytes(p)[:self.win_bytes].copy_(torch.from_numpy(raw))

    def window_bits(self, p):
        raw = self._bytes(p).cpu().numpy()
        w = raw[:self.win_bytes].view(np.uint16 if self.dtype == "bf16" else np.float32)
        return w.reshape(self.W - 1, self.C), raw[self.win_bytes:]


def run_conv(cp, x_dev, w_dev, cu, out_dtype, **kw):
    T = int(cu[-1])
    y = torch.full((T, cp.C), float("nan"), device="cuda",
                   dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    nck = 0 if kw.get("ckpt_cu") is None else int(kw["ckpt_cu"][-1])
    ws = torch.empty(max(256, K.kda_conv_workspace_bytes(len(cu) - 1, nck)), dtype=torch.uint8,
                     device="cuda")
    K.kda_short_conv(cp.pool, x_dev, w_dev, y, cu, workspace=ws, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def err_bound(x64, w64, cu, windows_in, out_dtype, ref):
    """Per-element bound: W fused multiply-adds in fp32 against the fp64 sum,
    plus one bf16 rounding of the fp32 result for bf16 outputs."""
    W = w64.shape[1]
    mag = np.zeros_like(ref)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        m, _ = conv.conv_segment(np.abs(x64[a:b]), np.abs(w64),
                                 None if windows_in[s] is None else np.abs(windows_in[s]))
        mag[a:b] = m
    fp32 = (W + 1) * U32 * mag + 1e-30
    return fp32 + (UBF * (np.abs(ref) + fp32) if out_dtype == "bf16" else 0.0)


def check_windows(cp, page, expect64, tag):
    got, tail = cp.window_bits(page)
    assert np.array_equal(got.view(np.uint8), to_bits(expect64, cp.dtype).view(np.uint8)), tag
    assert np.all(tail.view(np.int32) == POISON), f"{tag}: page tail overwritten"


# lens / starts: single token, ragged chunks, exactly one chunk, a boundary one
# token in, 512 crossed mid-block, two boundaries, empty sequences with and
# without an entering window.
LENS = [1, 63, 64, 65, 700, 1030, 0, 17, 0]
STARTS = [0, 5, 512, 448, 100, 1000, 30, 3, 0]
STATE_IN = [-1, 0, -1, 1, -1, 2, 3, -1, -1]


@pytest.mark.parametrize("dtype,out_dtype,W", [
    ("bf16", "bf16", 2), ("bf16", "bf16", 3), ("bf16", "bf16", 4),
    ("f32", "f32", 2), ("f32", "f32", 3), ("f32", "f32", 4), ("bf16", "f32", 3)])
def test_conv_parity_varlen(dtype, out_dtype, W):
    C = 2400 if dtype == "bf16" else 1200   # 300 channel groups: one full and one partial column
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    T = int(cu[-1])
    seed = 40 + W
    x = G.conv_inputs(seed, T, C, dtype)
    w = G.conv_weights(seed, C, W)
    x64, w64 = to64(x, dtype), w.astype(np.float64)
    wins = G.conv_inputs(seed + 1000, 4 * (W - 1), C, dtype)
    cp = ConvPool(40, C, W, dtype)
    windows_in = []
    for s, p in enumerate(STATE_IN):
        if p >= 0:
            v = to64(wins[p * (W - 1):(p + 1) * (W - 1)], dtype)
            cp.set_window(p, v)
            windows_in.append(v)
        else:
            windows_in.append(None)
    state_out = [-1] + [10 + s for s in range(1, len(LENS))]
    ckpts, ckpt_pages = [], []
    nxt = 25
    for s in range(len(LENS)):
        ps = [P for P in range(512, STARTS[s] + LENS[s] + 1, 512) if P > STARTS[s]]
        ckpts.append(ps)
        ckpt_pages.append(list(range(nxt, nxt + len(ps))))
        nxt += len(ps)
    assert sum(map(len, ckpts)) == 4
    ckpt_cu = np.concatenate([[0], np.cumsum([len(c) for c in ckpts])]).astype(np.int32)
    y = run_conv(cp, dev(x, dtype), torch.from_numpy(w).cuda(), cu, out_dtype,
                 start_pos=STARTS, state_in_page=STATE_IN, state_out_page=state_out,
                 ckpt_cu=ckpt_cu, ckpt_pos=[P for c in ckpts for P in c],
                 ckpt_page=[p for c in ckpt_pages for p in c])
    ref, finals, ck = conv.short_conv_varlen(x64, w64, cu, STARTS, windows_in, ckpts)
    bound = err_bound(x64, w64, cu, windows_in, out_dtype, ref)
    bad = np.abs(y - ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside the rounding bound, first at {np.argwhere(bad)[0]}"
    assert rel_fro(y, ref) <= (1e-5 if out_dtype == "f32" else 4e-3)
    for s in range(len(LENS)):
        if state_out[s] >= 0:
            check_windows(cp, state_out[s], finals[s], f"final window of sequence {s}")
        for P, pg, v in zip(ckpts[s], ckpt_pages[s], ck[s]):
            check_windows(cp, pg, v, f"checkpoint {P} of sequence {s}")
    # the empty sequence without an entering window leaves a zero window
    assert np.all(finals[8] == 0)
    # pages the call neither read nor wrote keep their poison
    written = {p for p in state_out if p >= 0} | {p for c in ckpt_pages for p in c}
    words = cp.buf.cpu().numpy().reshape(40, -1)
    for p in range(40):
        if p not in written and p not in STATE_IN:
            assert np.all(words[p] == POISON), f"page {p} touched"


def test_conv_split_and_resume_bitwise():
    """A sequence run in one call, in two calls joined by the window page, and
    resumed from its checkpoint window at 1024 gives identical bits."""
    dtype, W, C, T = "bf16", 4, 1024, 1500
    x = G.conv_inputs(7, T, C, dtype)
    w = torch.from_numpy(G.conv_weights(7, C, W)).cuda()
    xd = dev(x, dtype)
    cp = ConvPool(8, C, W, dtype)
    whole = run_conv(cp, xd, w, [0, T], "bf16", state_out_page=[0], ckpt_cu=[0, 2],
                     ckpt_pos=[512, 1024], ckpt_page=[1, 2])
    a = run_conv(cp, xd[:700], w, [0, 700], "bf16", state_out_page=[3])
    b = run_conv(cp, xd[700:], w, [0, T - 700], "bf16", start_pos=[700], state_in_page=[3],
                 state_out_page=[4])
    assert np.array_equal(np.concatenate([a, b]), whole)
    r = run_conv(cp, xd[1024:], w, [0, T - 1024], "bf16", start_pos=[1024], state_in_page=[2],
                 state_out_page=[5])
    assert np.array_equal(r, whole[1024:])
    for p in (4, 5):
        assert np.array_equal(cp.window_bits(p)[0], cp.window_bits(0)[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_decode_shape(dtype):
    """The decode-step update: 256 requests of one token each over the fused
    q|k|v channels (12,288), width 4, every request entering with its window
    page and writing its new window to a fresh page; requests whose token lands
    on a 512 boundary also write a checkpoint window.  Outputs within the
    rounding bound of the oracle, windows bit-exact, and three such steps
    (pages alternating) equal one 3-token call bit for bit."""
    W, C, n = 4, 3 * 32 * 128, 256
    if dtype == "f32":
        C //= 2
    rng = np.random.default_rng(17)
    starts = [int(x) for x in rng.integers(1, 4000, n)]
    for r in range(0, n, 37):
        starts[r] = 512 * (1 + r % 5) - 1  # the token ends at a 512 boundary
    cu = np.arange(n + 1, dtype=np.int64)
    x = G.conv_inputs(81, n, C, dtype)
    w = G.conv_weights(81, C, W)
    x64, w64 = to64(x, dtype), w.astype(np.float64)
    wins = G.conv_inputs(82, n * (W - 1), C, dtype)
    ck_req = [r for r in range(n) if (starts[r] + 1) % 512 == 0]
    cp = ConvPool(2 * n + len(ck_req), C, W, dtype)
    windows_in = []
    for r in range(n):
        v = to64(wins[r * (W - 1):(r + 1) * (W - 1)], dtype)
        cp.set_window(r, v)
        windows_in.append(v)
    ckpt_cu = np.zeros(n + 1, np.int32)
    for r in ck_req:
        ckpt_cu[r + 1:] += 1
    ckpt_pos = [starts[r] + 1 for r in ck_req]
    ckpt_page = [2 * n + i for i in range(len(ck_req))]
    y = run_conv(cp, dev(x, dtype), torch.from_numpy(w).cuda(), cu, dtype, start_pos=starts,
                 state_in_page=list(range(n)), state_out_page=list(range(n, 2 * n)),
                 ckpt_cu=ckpt_cu, ckpt_pos=ckpt_pos, ckpt_page=ckpt_page)
    ref, finals, ck = conv.short_conv_varlen(x64, w64, cu, starts, windows_in,
                                             [[starts[r] + 1] if r in ck_req else [] for r in range(n)])
    bound = err_bound(x64, w64, cu, windows_in, dtype, ref)
    assert not (np.abs(y - ref) > bound).any()
    for r in range(n):
        check_windows(cp, n + r, finals[r], f"window of request {r}")
    for i, r in enumerate(ck_req):
        check_windows(cp, 2 * n + i, ck[r][0], f"checkpoint window of request {r}")
    # three decode steps, pages alternating, against one 3-token call per request
    xs = G.conv_inputs(83, 3 * 8, C, dtype)
    wd = torch.from_numpy(w).cuda()
    cp2 = ConvPool(4 * 8, C, W, dtype)
    for r in range(8):  # pages 0-7 for the steps (rewritten by step 1), 24-31 for the single call
        cp2.set_window(r, windows_in[r])
        cp2.set_window(24 + r, windows_in[r])
    outs = []
    for t in range(3):
        xt = np.ascontiguousarray(xs.reshape(8, 3, C)[:, t])
        outs.append(run_conv(cp2, dev(xt, dtype), wd, np.arange(9, dtype=np.int64), dtype,
                             start_pos=[starts[r] + 1 + t for r in range(8)],
                             state_in_page=[(t % 2) * 8 + r for r in range(8)],
                             state_out_page=[((t + 1) % 2) * 8 + r for r in range(8)]))
    one = run_conv(cp2, dev(xs, dtype), wd, np.arange(0, 25, 3, dtype=np.int64), dtype,
                   start_pos=[starts[r] + 1 for r in range(8)], state_in_page=list(range(24, 32)),
                   state_out_page=list(range(16, 24)))
    assert np.array_equal(np.stack(outs, 1).reshape(24, C), one)
    for r in range(8):
        assert np.array_equal(cp2.window_bits(8 + r)[0], cp2.window_bits(16 + r)[0])


@pytest.mark.parametrize("dtype,W", [("bf16", 4), ("f32", 3), ("bf16", 2)])
def test_conv_update_matches_short_conv(dtype, W, monkeypatch):
    """kda_short_conv_update (device page tables, one token per request) gives
    the bits of kda_short_conv on the same 1-token sequences: y and the new
    windows; in place (page_out == page_in) as well; a request with a page
    index outside the pool gets NaN outputs and touches no page; outputs match
    the oracle within the rounding bound."""
    monkeypatch.delenv("KDA_VALIDATE", raising=False)  # the device-side handling is under test
    C, n = 3 * 32 * 128 // (1 if dtype == "bf16" else 2), 200
    x = G.conv_inputs(91 + W, n, C, dtype)
    w = G.conv_weights(91 + W, C, W)
    wins = G.conv_inputs(92 + W, n * (W - 1), C, dtype)
    wd = torch.from_numpy(w).cuda()
    xd = dev(x, dtype)
    cp = ConvPool(3 * n + 1, C, W, dtype)
    win64 = [to64(wins[r * (W - 1):(r + 1) * (W - 1)], dtype) for r in range(n)]
    for r in range(n):
        cp.set_window(r, win64[r])
        cp.set_window(2 * n + r, win64[r])
    ref_y = run_conv(cp, xd, wd, np.arange(n + 1, dtype=np.int64), dtype, start_pos=[7] * n,
                     state_in_page=list(range(n)), state_out_page=list(range(n, 2 * n)))
    # out of place: windows 0..n-1 -> fresh pages (the last request's page is invalid)
    cp2 = ConvPool(3 * n + 1, C, W, dtype)
    for r in range(n):
        cp2.set_window(r, win64[r])
    before = cp2.buf.cpu().numpy().copy()
    y = torch.full((n, C), float("nan"), device="cuda",
                   dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    pout = torch.arange(n, 2 * n, dtype=torch.int32, device="cuda")
    pout[n - 1] = 3 * n + 5  # outside the pool
    K.kda_short_conv_update(cp2.pool, xd, wd, y, pin, pout)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:n - 1], ref_y[:n - 1])
    assert np.all(np.isnan(got[n - 1]))
    for r in range(n - 1):
        assert np.array_equal(cp2.window_bits(n + r)[0], cp.window_bits(n + r)[0]), r
    after = cp2.buf.cpu().numpy().reshape(3 * n + 1, -1)
    assert np.array_equal(after[2 * n - 1:], before.reshape(3 * n + 1, -1)[2 * n - 1:])
    assert np.array_equal(after[:n], before.reshape(3 * n + 1, -1)[:n])  # inputs unchanged
    # in place on pages 2n .. 3n-1
    y2 = torch.empty_like(y)
    pio = torch.arange(2 * n, 3 * n, dtype=torch.int32, device="cuda")
    K.kda_short_conv_update(cp.pool, xd, wd, y2, pio, pio)
    torch.cuda.synchronize()
    assert np.array_equal(y2.float().cpu().numpy().astype(np.float64), ref_y)
    for r in range(n):
        assert np.array_equal(cp.window_bits(2 * n + r)[0], cp.window_bits(n + r)[0]), r
    # against the oracle
    x64, w64 = to64(x, dtype), w.astype(np.float64)
    cu = np.arange(n + 1)
    ref, finals, _ = conv.short_conv_varlen(x64, w64, cu, [7] * n, win64)
    bound = err_bound(x64, w64, cu, win64, dtype, ref)
    assert not (np.abs(ref_y - ref) > bound).any()
    for r in range(n):
        check_windows(cp, n + r, finals[r], f"window of request {r}")


def test_conv_full_size_8k():
    """The bench workload: the fused q|k|v projection of 8192 tokens
    (3 x 32 heads x 128 channels), width 4, a checkpoint at every 512-token
    boundary."""
    dtype, W, C, T = "bf16", 4, 3 * 32 * 128, 8192
    x = G.conv_inputs(3, T, C, dtype)
    w = G.conv_weights(3, C, W)
    cp = ConvPool(20, C, W, dtype, extra=0)
    P = list(range(512, T + 1, 512))
    y = run_conv(cp, dev(x, dtype), torch.from_numpy(w).cuda(), [0, T], "bf16",
                 state_out_page=[0], ckpt_cu=[0, len(P)], ckpt_pos=P,
                 ckpt_page=list(range(1, 1 + len(P))))
    x64, w64 = to64(x, dtype), w.astype(np.float64)
    ref, finals, ck = conv.short_conv_varlen(x64, w64, [0, T], None, None, [P])
    bound = err_bound(x64, w64, [0, T], [None], "bf16", ref)
    assert not (np.abs(y - ref) > bound).any()
    got, _ = cp.window_bits(0)
    assert np.array_equal(got, to_bits(finals[0], dtype))
    for i, v in enumerate(ck[0]):
        assert np.array_equal(cp.window_bits(1 + i)[0], to_bits(v, dtype)), f"checkpoint {P[i]}"


def test_conv_update_validate_mode(monkeypatch):
    """With KDA_VALIDATE=1 kda_short_conv_update reads the page tables back and
    checks them on the host first: a valid call gives the bits of the unchecked
    one; an index outside the pool, a repeated output page and an input page
    that is another request's output are rejected with the documented status,
    and no page or output changes."""
    dtype, W, C, n = "bf16", 4, 2048, 8
    x = G.conv_inputs(17, n, C, dtype)
    w = G.conv_weights(17, C, W)
    wins = G.conv_inputs(18, n * (W - 1), C, dtype)
    xd, wd = dev(x, dtype), torch.from_numpy(w).cuda()

    def fresh():
        cp = ConvPool(2 * n, C, W, dtype)
        for r in range(n):
            cp.set_window(r, to64(wins[r * (W - 1):(r + 1) * (W - 1)], dtype))
        return cp

    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    pout = torch.arange(n, 2 * n, dtype=torch.int32, device="cuda")
    runs = []
    for val in (None, "1"):
        if val is None:
            monkeypatch.delenv("KDA_VALIDATE", raising=False)
        else:
            monkeypatch.setenv("KDA_VALIDATE", val)
        cp = fresh()
        y = torch.empty((n, C), dtype=torch.bfloat16, device="cuda")
        K.kda_short_conv_update(cp.pool, xd, wd, y, pin, pout)
        torch.cuda.synchronize()
        runs.append((y.view(torch.int16).cpu(), cp.buf.cpu()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])

    def with_(t, i, val):
        t = t.clone()
        t[i] = val
        return t

    for bad_in, bad_out, status in [
            (with_(pin, 2, 2 * n + 3), pout, K.KDA_ERR_PAGE_RANGE),
            (pin, with_(pout, 5, -1), K.KDA_ERR_PAGE_RANGE),
            (pin, with_(pout, 7, n), K.KDA_ERR_PAGE_ALIAS),       # output page n twice
            (with_(pin, 1, n), pout, K.KDA_ERR_PAGE_ALIAS)]:      # request 0's output read by request 1
        cp = fresh()
        before = cp.buf.clone()
        y = torch.full((n, C), 3.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(K.KdaError) as e:
            K.kda_short_conv_update(cp.pool, xd, wd, y, bad_in, bad_out)
        assert e.value.status == status, (e.value, status)
        torch.cuda.synchronize()
        assert torch.equal(cp.buf, before) and bool(torch.all(y == 3.0))
