"""GPU parity of the forward on T axes past what one item can address (T >= 2^22 tokens):
the segment plan then cuts every sequence into items of at most 2^21 tokens.

The oracle cannot run millions of tokens per test, so windows are checked through a property
of the recurrence. A run of L tokens with the floor decay g = -5 on every channel maps the state
entering it to A S + B: B is what the run's own tokens write, and A is the product of the
tokens' maps (I - beta k k^T) Diag(e^g). With unit keys and beta in [0, 1] each (I - beta k k^T)
has norm at most 1 (at most 2 for the Gated Delta Rule-2 factor I - k (b * k)^T), and Diag(e^g)
has norm e^-5, so |A| <= 2^L e^(-5 L). For L = 32 that is below 1e-60: far under bf16 rounding.
The outputs after such a run therefore equal those of the same tokens started from the zero
state at the run's first token, which the oracle computes in a few thousand steps. Windows
across the plan's segment boundaries, across the former whole-chain bound (2^22 tokens) and at
the end of the axis are checked that way. The first tokens are checked from the true initial
state, and the final state is checked from the last window.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
import oracle
from kda_workloads import make_long_chain_inputs, set_floor
from tests.gpu_util import TOL, assert_close, dev, note

pytestmark = pytest.mark.gpu

RUN = 32      # tokens of floor decay before a window
LEAD = 3000   # tokens from the start of the run to the window
WIN = 1000    # tokens checked per window
DK = DV = 128


def call(x, cu, N, H, T):
    """One forward call with the recommended workspace. Returns (o, final state, the plan's
    five header words: [0] items, [1] segment length in 64-token chunks, [2] slots,
    [3] correction units and [4] carried-back-query rows per head)."""
    num = N if cu is not None else 0
    nbytes = kda.kda_chunk_fwd_workspace_size(1, H, T, DK, DV, num, kda.KDA_BF16)
    assert nbytes > 0, "no segment plan for the long axis"
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    o = torch.full((1, H, T, DV), float("nan"), dtype=torch.bfloat16, device=dev())
    sT = torch.empty((N, H, DK, DV), dtype=torch.float32, device=dev())
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    gm = kda.KDA_GATE_PER_CHANNEL if x.g.dim() == 4 else kda.KDA_GATE_PER_HEAD
    head = (ptr(x.q), ptr(x.k), ptr(x.v), ptr(x.g))
    tail = (ptr(x.s0), ptr(sT), ptr(o), ptr(cu), num, 1, H, T, DK, DV, kda.KDA_BF16,
            gm, ptr(ws), nbytes, torch.cuda.current_stream().cuda_stream)
    if x.erase is not None:
        st = kda.kda_gdr2_chunk_fwd(*head, ptr(x.erase), ptr(x.write), *tail)
    else:
        st = kda.kda_chunk_fwd(*head, ptr(x.beta), *tail)
    assert st == kda.KDA_OK, kda.kda_status_string(st)
    torch.cuda.synchronize()
    return o, sT, ws[:20].cpu().numpy().view(np.uint32).copy()


def oracle_span(x, h, a, b, s0=None):
    """The oracle on tokens a .. b - 1 of head h, from s0 [dk, dv] or the zero state."""
    host = lambda t: None if t is None else t[:, h:h + 1, a:b].float().cpu().numpy()  # noqa: E731
    beta = host(x.beta) if x.beta is not None else np.zeros((1, 1, b - a), np.float32)
    ref = oracle.kda_forward(host(x.q), host(x.k), host(x.v), host(x.g), beta,
                             s0=None if s0 is None else s0[None, None],
                             erase=host(x.erase), write=host(x.write))
    return ref[(0, 0)]


def check_window(x, o, h, w0, w1, what, s0=None, start=None):
    """Outputs of tokens w0 .. w1 - 1 against the oracle run from `start` (a run of floor
    decay placed there) or, with s0, from a sequence start at w0."""
    a = w0 if start is None else start
    ro, rs = oracle_span(x, h, a, w1, s0)
    got = o[0, h, w0:w1].float().cpu().numpy()
    e = assert_close(got, ro[w0 - a:], TOL["bf16"], what)
    note(f"{what}: normwise error {e:.2e}")
    return rs


def windows(seq_start, seq_len, xt, extra=()):
    """Windows (first token, end) inside one sequence: across each of its first, second and
    last segment boundaries, around the positions in `extra` (absolute tokens), and its last
    WIN tokens; each far enough from the sequence start for its run of floor decay."""
    ns = -(-seq_len // xt)
    cuts = sorted({xt, 2 * xt, (ns - 1) * xt} - {0})
    centres = [seq_start + c for c in cuts if c < seq_len] + list(extra)
    out = []
    for c in centres:
        w0 = c - WIN // 5
        if w0 - LEAD >= seq_start and w0 + WIN <= seq_start + seq_len:
            out.append((w0, w0 + WIN))
    out.append((seq_start + seq_len - WIN, seq_start + seq_len))
    return sorted(set(out))


@pytest.mark.parametrize("kind", ["kda", "gdr2", "gdn"])
def test_long_single_sequence(kind):
    """One sequence of 2^22 + 3000 tokens (two heads, random initial state), with KDA, Gated
    Delta Rule-2 or one decay per head (Gated DeltaNet): every output is written, the plan
    cuts it into items within the bound, and windows across its segment boundaries, the
    former whole-chain bound and its end match the oracle, as does the final state."""
    H, T = 2, (1 << 22) + 3000
    note(f"long chain: one sequence of {T} tokens, H={H}, {kind}")
    x = make_long_chain_inputs(T, H, seed=4101 + ["kda", "gdr2", "gdn"].index(kind), device=dev(),
                               gdr2=kind == "gdr2", gate="head" if kind == "gdn" else "channel")
    # the plan's segment length depends on the lengths only: learn it from a first call, which
    # also checks the first tokens from the true initial state
    o, _, hdr = call(x, None, 1, H, T)
    xc, slots = int(hdr[1]), int(hdr[2])
    note(f"long chain plan: {hdr[0]} items, segments of {xc} chunks, {slots} slots")
    assert 0 < xc <= (1 << 21) // 64 and slots >= -(-T // (64 * xc))
    assert bool(torch.isfinite(o).all()), "some output position was not written"
    s0 = x.s0.cpu().numpy()
    for h in range(H):
        check_window(x, o, h, 0, WIN, f"head {h} tokens 0..{WIN} from the initial state",
                     s0=s0[0, h])
    del o
    ws_ = windows(0, T, 64 * xc, extra=[1 << 22])
    for (w0, _) in ws_:
        set_floor(x.g, w0 - LEAD, RUN)
    o, sT, hdr2 = call(x, None, 1, H, T)
    assert np.array_equal(hdr, hdr2)
    for h in range(H):
        for (w0, w1) in ws_:
            rs = check_window(x, o, h, w0, w1, f"head {h} tokens {w0}..{w1}",
                              start=w0 - LEAD)
        assert_close(sT[0, h].cpu().numpy(), rs, TOL["bf16"], f"head {h} final state")


def test_long_packed_sequences():
    """Packed: a short sequence, one of 2^22 + 1500 tokens and a short one after it (one
    head). The short ones match the oracle whole; the long one in windows as above."""
    H = 1
    lens = [1000, (1 << 22) + 1500, 2500]
    T = sum(lens)
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(cu_h).to(dev())
    note(f"long chain: packed lengths {lens}")
    x = make_long_chain_inputs(T, H, seed=4111, device=dev(), n_seqs=len(lens))
    _, _, hdr = call(x, cu, len(lens), H, T)
    xc = int(hdr[1])
    note(f"long packed plan: {hdr[0]} items, segments of {xc} chunks, {hdr[2]} slots")
    assert 0 < xc <= (1 << 21) // 64
    ws_ = windows(int(cu_h[1]), lens[1], 64 * xc, extra=[1 << 22])
    for (w0, _) in ws_:
        set_floor(x.g, w0 - LEAD, RUN)
    o, sT, _ = call(x, cu, len(lens), H, T)
    assert bool(torch.isfinite(o).all()), "some output position was not written"
    s0 = x.s0.cpu().numpy()
    for n in (0, 2):
        a, b = int(cu_h[n]), int(cu_h[n + 1])
        rs = check_window(x, o, 0, a, b, f"short sequence {n} (tokens {a}..{b})", s0=s0[n, 0])
        assert_close(sT[n, 0].cpu().numpy(), rs, TOL["bf16"], f"sequence {n} final state")
    for (w0, w1) in ws_:
        rs = check_window(x, o, 0, w0, w1, f"long sequence tokens {w0}..{w1}", start=w0 - LEAD)
    assert_close(sT[1, 0].cpu().numpy(), rs, TOL["bf16"], "long sequence final state")
