"""Several host threads calling the library at once, each on its own stream:
the library promises that calls are safe from several host threads on
different streams (its state is per-device caches and per-kernel attribute
flags), and its kernels are deterministic for a given shape.  So every
thread's results must equal, bit for bit, the same calls made from one
thread.  The calls cover the M = 1 matvecs (f32 input), the group launch
and the small-M matmul with a workspace per thread."""
import threading

import pytest
import torch

import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import dev

pytestmark = pytest.mark.gpu
Q4, Q6 = kq.KQ_QTYPE_Q4K, kq.KQ_QTYPE_Q6K
NTHR, ITERS = 4, 6
N4, K4 = 2048, 6656
N6, K6 = 1536, 4096
NM, KM, M = 1000, 2560, 5
GROUP = [512, 64, 64, 512]


def calls(Ws, x4, x6, Xm, ws, stream):
    """One thread's work; returns its outputs (allocated on `stream`)."""
    W4, W6, Wm, Wg = Ws
    with torch.cuda.stream(stream):
        y4 = torch.empty(N4, device="cuda")
        y6 = torch.empty(N6, device="cuda")
        Y = torch.empty((M, NM), device="cuda")
        yg = [torch.empty(n, device="cuda") for n in GROUP]
        for _ in range(ITERS):
            kq.kq_matvec_q4k(W4, x4, y4, N4, K4, stream=stream)
            kq.kq_matvec_q6k(W6, x6, y6, N6, K6, stream=stream)
            kq.kq_matvec_group(Q4, Wg, yg, GROUP, x4, K4, stream=stream)
            kq.kq_matmul_small_m(Q4, Wm, Xm, KM, Y, NM, NM, KM, M, ws[0], ws[1], stream=stream)
    stream.synchronize()
    return [y4.cpu(), y6.cpu(), Y.cpu()] + [t.cpu() for t in yg]


def test_threads_on_separate_streams_give_single_thread_bits():
    Ws = (dev(I.q4k_matrix(N4, K4, stream=9100)), dev(I.q6k_matrix(N6, K6, stream=9101)),
          dev(I.q4k_matrix(NM, KM, stream=9102)),
          [dev(I.q4k_matrix(n, K4, stream=9103 + i)) for i, n in enumerate(GROUP)])
    x4 = [dev(I.normal_f32(K4, stream=9110 + t)) for t in range(NTHR)]
    x6 = [dev(I.normal_f32(K6, stream=9120 + t)) for t in range(NTHR)]
    Xm = [dev(I.normal_f32((M, KM), stream=9130 + t)) for t in range(NTHR)]
    need = kq.kq_matmul_small_m_workspace_bytes(Q4, NM, KM, M)
    wss = [(torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda"), need)
           for _ in range(NTHR + 1)]
    torch.cuda.synchronize()
    # reference: one thread, the calls in sequence
    ref = [calls(Ws, x4[t], x6[t], Xm[t], wss[NTHR], torch.cuda.Stream()) for t in range(NTHR)]
    # every thread at once, each with its own stream and workspace
    out, errors = [None] * NTHR, []

    def run(t):
        try:
            out[t] = calls(Ws, x4[t], x6[t], Xm[t], wss[t], torch.cuda.Stream())
        except Exception as e:  # reported below; an exception in a thread would be lost
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=run, args=(t,)) for t in range(NTHR)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(NTHR):
        for i, (a, b) in enumerate(zip(out[t], ref[t])):
            assert torch.isfinite(b).all(), f"thread {t} output {i}: reference not finite"
            assert torch.equal(a, b), f"thread {t} output {i} differs from the single-thread bits"
