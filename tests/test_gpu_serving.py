"""End to end on the GPU: the host step planner (libpa pa_sched_*) drives pa_append_kv and
pa_attention over many steps -- chunked prompts interleaved with decodes (P4 "一步的 token 预算"),
shared-prefix hits that reuse cached blocks written by other requests (P3 §4.3), evictions and
recompute preemption in a small pool -- and every step's output is compared with the oracle run
from scratch on a fresh contiguous cache per request (see tests/serving_helpers.py).
"""
import numpy as np
import pytest
import torch

import attention_paged_kv_amd as pa
from tests.gpu_helpers import DEV, compare, host_array, say
from tests.serving_helpers import D, HKV, drive

pytestmark = pytest.mark.gpu


class GpuExecutor:
    def __init__(self, nb):
        self.kc = torch.zeros((nb, 16, HKV, D), dtype=torch.bfloat16, device=DEV)
        self.vc = torch.zeros_like(self.kc)

    def __call__(self, b, q, kn, vn, scale):
        bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
        dq, dk, dv = bf(q), bf(kn), bf(vn)
        pa.append_kv(dk, dv, torch.from_numpy(b.slot_mapping).to(DEV), self.kc, self.vc)
        out = torch.empty_like(dq)
        pa.attention(dq, self.kc, self.vc, torch.from_numpy(b.block_tables).to(DEV),
                     torch.from_numpy(b.seq_lens).to(DEV), torch.from_numpy(b.query_start_loc).to(DEV), scale, out)
        torch.cuda.synchronize()
        return host_array(out, "bf16")


@pytest.mark.parametrize("seed,nb,budget,prefix", [(0, 40, 96, True), (1, 18, 64, True), (2, 40, 96, False)])
def test_planner_drives_the_kernels_end_to_end(seed, nb, budget, prefix):
    def check(out, ref, step, b):
        say(f"seed {seed} step {step}: B={b.num_seqs} T={b.num_tokens}")
        compare(out, ref, "bf16", what=f"serving step {step}")
    c = drive(seed, nb, budget, prefix, GpuExecutor(nb), check)
    say(f"counters {c}")
    assert c["steps"] > 20
    if prefix:
        assert c["hits"] > 0
    if nb < 20:
        assert c["preempts"] > 0
