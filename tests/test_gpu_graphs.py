"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed several times, with eager work and synchronizations between the
replays: each replay's outputs must equal the eager call's, bit for bit.
And entry points on two streams at once give the bytes of a sequential run."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _replay_check(fn, outs, replays=4):
    """fn() writes into the tensors `outs`; eager result first, then a captured
    graph replayed `replays` times, the outputs scrambled before each replay.
    An entry of `outs` may be (tensor, mask): only the masked elements are
    written by fn and compared."""
    masks = [o[1] if isinstance(o, tuple) else None for o in outs]
    outs = [o[0] if isinstance(o, tuple) else o for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    junk = torch.empty(1 << 20, device="cuda").uniform_()
    for k in range(replays):
        for o in outs:                            # eager work between replays
            o.view(torch.uint8).fill_(0x5A + k)
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r, mk in zip(outs, ref, masks):
            if mk is not None:
                o, r = o[mk], r[mk]
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {k} differs"


def test_graphs_of_every_entry_point():
    m = need_gpu()
    torch.manual_seed(0)
    x = (torch.randn((512, 1024), device="cuda") * 3).to(torch.bfloat16)
    xf = torch.randn((512, 1024), device="cuda")
    # NVFP4 with the tensor scale computed (three kernels) and given; MXFP4
    for fmt, tscale in (("nvfp4", "compute"), ("nvfp4", "given"), ("mxfp4", "compute")):
        blk = 16 if fmt == "nvfp4" else 32
        p = torch.empty((512, 512), dtype=torch.uint8, device="cuda")
        s = torch.empty((512, 1024 // blk), dtype=torch.uint8, device="cuda")
        ts = torch.tensor([1.5e-3], dtype=torch.float32, device="cuda")
        y = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")
        outs = [p, s, y] + ([ts] if fmt == "nvfp4" and tscale == "compute" else [])

        def fn(fmt=fmt, tscale=tscale, p=p, s=s, ts=ts, y=y):
            m.fp4_quantize(x, fmt, "sr", seed=7, step=3, tscale=tscale,
                           tensor_scale=ts if fmt == "nvfp4" else None, packed=p, scales=s)
            m.fp4_dequantize(p, s, 512, 1024, fmt, ts if fmt == "nvfp4" else None, y=y)
        _replay_check(fn, outs)
    # FP4Quant
    p = torch.empty((512, 512), dtype=torch.uint8, device="cuda")
    s1 = torch.empty((512, 16), dtype=torch.float32, device="cuda")
    s2 = torch.empty((512, 16), dtype=torch.float32, device="cuda")
    yq = torch.empty((512, 1024), dtype=torch.float32, device="cuda")

    def fq():
        m.fp4quant_encode(x, 64, p, s1, s2)
        m.fp4quant_decode(p, s1, s2, 512, 1024, 64, torch.float32, yq)
    _replay_check(fq, [p, s1, s2, yq])
    # the FP4Quant SR variant (G = 256: the four-lane row layout)
    s1b = torch.empty((512, 4), dtype=torch.float32, device="cuda")
    s2b = torch.empty((512, 4), dtype=torch.float32, device="cuda")

    def fqs():
        m.fp4quant_encode_ex(x, 256, "sr", 5, 8, p, s1b, s2b)
    _replay_check(fqs, [p, s1b, s2b])
    # error feedback (computed scale, the residual restored before each run)
    r0 = torch.randn((512, 1024), device="cuda") * 1e-3
    r = r0.clone()
    w = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    pe = torch.empty((512, 512), dtype=torch.uint8, device="cuda")
    se = torch.empty((512, 64), dtype=torch.uint8, device="cuda")

    def ef():
        r.copy_(r0)
        m.fp4_errfeedback_qdq(xf, r, w, None, "sr", 9, 2, "compute", ts, pe, se)
    _replay_check(ef, [r, w, ts, pe, se])

    def ef_nocodes():                               # partial maxima kept in w
        r.copy_(r0)
        m.fp4_errfeedback_qdq(xf, r, w, None, "sr", 9, 2, "compute", ts)
    _replay_check(ef_nocodes, [r, w, ts])
    # FP8 rows and columns over ragged experts
    T, H = 3000, 768
    counts = np.random.default_rng(3).integers(0, 120, size=40)
    counts[-1] = T - counts[:-1].sum() if T > counts[:-1].sum() else 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    pk, sb = synth.random_mxfp4(T, H, seed=4)
    pk, sb, offd = torch.from_numpy(pk).cuda(), torch.from_numpy(sb).cuda(), torch.from_numpy(off).cuda()
    o8 = torch.empty(T * H, dtype=torch.uint8, device="cuda")
    s8 = torch.empty(T * H // 128, dtype=torch.float32, device="cuda")
    o8r = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    s8r = torch.empty((T, H // 128), dtype=torch.float32, device="cuda")

    o8t = torch.empty(T * H, dtype=torch.uint8, device="cuda")
    s8t = torch.zeros(m.tokblk_scale_count(T, off.size - 1, H), dtype=torch.float32, device="cuda")
    # the scale entries the call writes: expert e's [H, ceil(n_e/128)] at H (ceil(off_e/128) + e)
    wmask = torch.zeros(s8t.numel(), dtype=torch.bool)
    for e in range(off.size - 1):
        n = int(off[e + 1] - off[e])
        base = H * (-(-int(off[e]) // 128) + e)
        wmask[base: base + H * (-(-n // 128))] = True
    wmask = wmask.cuda()

    def f8():
        m.mxfp4_row_to_fp8_col(pk, sb, offd, H, o8, s8)
        m.mxfp4_row_to_fp8_col_tokblk(pk, sb, offd, H, o8t, s8t)
        m.mxfp4_row_to_fp8_row(pk, sb, H, o8r, s8r)
    _replay_check(f8, [o8, s8, o8t, (s8t, wmask), o8r, s8r])


def test_two_streams_at_once():
    """Entry points launched on two non-default streams (default priority)
    at the same time give the bytes of the same calls run one after another
    on the default stream: every call keeps to its own buffers and stream."""
    m = need_gpu()
    torch.manual_seed(1)
    x = (torch.randn((2048, 7168), device="cuda") * 2).to(torch.bfloat16)
    T, H = 4096, 1024
    counts = np.random.default_rng(8).integers(0, 40, size=128)
    counts[-1] += T - counts.sum() if T > counts.sum() else 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    pk, sb = synth.random_mxfp4(T, H, seed=8)
    pk, sb, offd = torch.from_numpy(pk).cuda(), torch.from_numpy(sb).cuda(), torch.from_numpy(off).cuda()

    def run(sa, sb_):
        outs = {}
        with torch.cuda.stream(sa):
            p, s, _ = m.fp4_quantize(x, "mxfp4", "rtn", stream=sa)
            outs["y"] = m.fp4_dequantize(p, s, 2048, 7168, "mxfp4", stream=sa)
            outs["p"], outs["s"] = p, s
        with torch.cuda.stream(sb_):
            outs["o8"], outs["s8"] = m.mxfp4_row_to_fp8_col(pk, sb, offd, H, stream=sb_)
            outs["o8r"], outs["s8r"] = m.mxfp4_row_to_fp8_row(pk, sb, H, stream=sb_)
            nst = m.tokblk_scale_count(T, off.size - 1, H)
            outs["o8t"], outs["s8t"] = m.mxfp4_row_to_fp8_col_tokblk(
                pk, sb, offd, H, fp8_scales=torch.zeros(nst, dtype=torch.float32, device="cuda"), stream=sb_)
            outs["q"], _, _ = m.fp4quant_encode_ex(x, 256, "sr", 3, 4, stream=sb_)
        torch.cuda.synchronize()
        return outs

    d = torch.cuda.current_stream()
    ref = run(d, d)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        got = run(s1, s2)
        for k in ref:
            assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), k
