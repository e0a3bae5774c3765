"""A process that loads libi8kv.so before it imports torch (the library then
brings torch's HIP runtime in first) runs a chunk-sized producer call and a
decode correctly: the producer's codes and scales equal those of the same call
in this (torch-first) process, bit for bit."""
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu
ROOT = Path(__file__).resolve().parent.parent

CHILD = r'''
import sys
sys.path.insert(0, sys.argv[1])
import int8_kv_quantized_amd as K
K.load_library()                      # before any torch import in this process
import numpy as np
import torch
import workloads as W
wl = W.make_workload("load_order", seq_lens=(4100,), new_tokens=(1,), num_q_heads=24,
                     num_kv_heads=4, head_dim=256, seed=97)
d = K.CacheDesc(24, 4, 256, wl.num_blocks)
c = K.PagedCache.allocate(d)
dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
K.kv_quantize_write(d, dev(wl.key), dev(wl.value), dev(wl.slot_mapping), c)
torch.cuda.synchronize()
np.savez(sys.argv[2], k=c.k_cache.cpu().numpy(), v=c.v_cache.cpu().numpy(),
         ks=c.k_scale.cpu().numpy(), vs=c.v_scale.cpu().numpy())
print("child ok")
'''


def test_library_loaded_before_torch(tmp_path):
    import int8_kv_quantized_amd as K
    import torch
    import workloads as W
    say("  load order: child process loads the library before torch")
    out = tmp_path / "child.npz"
    r = subprocess.run([sys.executable, "-c", CHILD, str(ROOT), str(out)], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0 and "child ok" in r.stdout, r.stderr[-3000:]
    wl = W.make_workload("load_order", seq_lens=(4100,), new_tokens=(1,), num_q_heads=24,
                         num_kv_heads=4, head_dim=256, seed=97)
    d = K.CacheDesc(24, 4, 256, wl.num_blocks)
    c = K.PagedCache.allocate(d)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    K.kv_quantize_write(d, dev(wl.key), dev(wl.value), dev(wl.slot_mapping), c)
    torch.cuda.synchronize()
    got = np.load(out)
    for name, t in (("k", c.k_cache), ("v", c.v_cache), ("ks", c.k_scale), ("vs", c.v_scale)):
        a, b = got[name], t.cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name} differs"
