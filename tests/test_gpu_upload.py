"""The plan upload only enqueues work: it does not wait for the device.

Every call of the library only enqueues on the caller's stream. The plan
upload stages its tables in page-locked slots; a slot whose copy has not run
yet is skipped and the ring grows, so even 40 uploads queued behind a long
kernel return at once, and each one still delivers its own plan.
"""
import sys
import time

import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_uploads_behind_a_long_kernel_do_not_block():
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    w = W.WORKLOADS["dcs_8k"]
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    # Different plans (rank, layout), so each upload's bytes are its own.
    plans = [thd.Plan(cu, cup, w.T, w.cp_size, i % 2, w.strategy, w.H, w.D, upload=False,
                      kv_layout=("rank_major" if (i // 2) % 2 else "global"))
             for i in range(40)]
    nbytes = max(int(p.info.workspace_bytes) for p in plans) + 256
    ws = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in plans]
    ref = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in plans]
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # Reference images: each plan uploaded with the device idle.
    for p, r in zip(plans, ref):
        p.upload_into(r, stream)
        torch.cuda.synchronize()

    # A long queue of device work (~tens of ms of matmuls), then 40 uploads.
    ev_busy = torch.cuda.Event()
    b = a
    for _ in range(24):
        b = a @ b
    ev_busy.record(stream)
    t0 = time.perf_counter()
    for p, x in zip(plans, ws):
        p.upload_into(x, stream)
    host_s = time.perf_counter() - t0
    busy_when_done = not ev_busy.query()
    ev_end = torch.cuda.Event(enable_timing=True)
    ev_end.record(stream)
    torch.cuda.synchronize()
    _say(f"40 uploads queued in {host_s * 1e3:.2f} ms of host time; "
         f"device still busy with the matmuls when they returned: {busy_when_done}")
    # The matmuls were still running when the last upload returned: none of
    # the 40 calls waited for the device.
    assert busy_when_done
    for i, (x, r) in enumerate(zip(ws, ref)):
        assert torch.equal(x, r), f"upload {i} delivered other bytes"
    for p in plans:
        p.close()
    del b
