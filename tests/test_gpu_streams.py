"""Copies issued from several host threads at once, each thread on its own HIP stream (default
priority): every result equals the oracle's, and a strict-mode decline planned in one thread
carries its own reason while the other threads' copies run."""

import threading

import numpy as np
import pytest

import layout_permuting_copy_amd as L
from gpu_util import oracle_copy, say

pytestmark = pytest.mark.gpu

DT = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}
# (rows, cols) transposed, element bytes: LDS tile plans of every width, ragged edges included
CASES = [((1536, 2048), 4), ((1000, 3000), 2), ((2047, 1023), 1), ((512, 4096), 8), ((300, 700), 16),
         ((4096, 512), 4), ((777, 1500), 1), ((1024, 1024), 2)]


def test_copies_from_threads_on_separate_streams():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    jobs = []
    for t, ((n, m), eb) in enumerate(CASES):
        src = np.frombuffer(np.random.default_rng(100 + t).bytes(n * m * eb), dtype=np.uint8).copy()
        sl, dl = ((n, m), (m, 1), 0), ((n, m), (1, n), 0)
        jobs.append((src, sl, dl, eb, oracle_copy(src, sl, n * m, dl, eb)))
    say(f"[gpu] {len(jobs)} threads, one stream each, 4 copies per thread")
    errors, done = [], [0] * len(jobs)

    def worker(i):
        try:
            src, sl, dl, eb, want = jobs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                src_d = torch.from_numpy(src).to("cuda")
                for rep in range(4):
                    dst_d = torch.full((want.size,), 0xA5, dtype=torch.uint8, device="cuda")
                    L.tile_copy(src_d, sl, dst_d, dl, DT[eb], stream=s.cuda_stream)
                    p = L.tc_plan(((1001, 37), (37, 1)), ((1001, 37), (1, 1001)), DT[eb], flags=L.TC_FLAG_STRICT,
                                  raise_on_error=False)
                    if p["status"] != L.TC_E_DECLINED or "64" not in p["error"]:
                        errors.append((i, rep, "decline", p["status"], p["error"]))
                    s.synchronize()
                    got = dst_d.cpu().numpy()
                    if not np.array_equal(got, want):
                        errors.append((i, rep, "bytes differ", int(np.count_nonzero(got != want))))
                        return
                    done[i] += 1
        except Exception as e:  # reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors[:4]
    assert done == [4] * len(jobs)
