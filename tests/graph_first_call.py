"""Child process of test_gpu_8_graph.test_first_decode_call_inside_capture.

In a fresh process, the first decode call of the library is made inside a HIP
graph capture: pa_decode_append_noalloc, whose callers cannot allocate (code
under graph capture among them). Its one-time set-up (the device's compute
units, the decode kernel's occupancy and the address of the fixed workspace)
therefore runs during the capture. The graph is replayed twice, and its output
and pools must equal, bit for bit, those of pa_decode_append launched
eagerly afterwards on a second pair of pools. Prints one line and exits 0 on
success.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import paged_kv_cache_245_amd as pa  # noqa: E402
import workloads  # noqa: E402
from gpu_support import device_tensor, gpu_pools, i32  # noqa: E402


def bits(t):
    return t.view(torch.int16).cpu().numpy()


def main():
    print("  first decode call inside a graph capture", flush=True)
    w = workloads.custom_decode(31, [1, 16, 17, 40, 300, 1111, 70, 9], Hq=32, Hkv=8, D=128, dtype="bf16")
    d, k0, v0 = gpu_pools(w, include_step=False)
    dec, sw = w.decode, w.step_write
    q = device_tensor(dec.q, "bf16")
    key, value = device_tensor(sw.key, "bf16"), device_tensor(sw.value, "bf16")
    tables, lens = i32(dec.block_tables), i32(dec.context_lens)
    S = len(dec.context_lens)

    kg, vg = k0.clone(), v0.clone()
    out_g = torch.zeros_like(q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pa.pa_decode_append_noalloc(d, out_g, q, key, value, kg, vg, tables, lens, dec.max_context_len, w.scale)
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()

    ke, ve = k0.clone(), v0.clone()
    out_e = torch.zeros_like(q)
    ws = pa.decode_workspace(d, S, dec.max_context_len)
    pa.pa_decode_append(d, out_e, q, key, value, ke, ve, tables, lens, dec.max_context_len, w.scale, ws)
    torch.cuda.synchronize()

    assert np.array_equal(bits(out_g), bits(out_e)), "replayed output differs from the eager call"
    assert np.array_equal(bits(kg), bits(ke)) and np.array_equal(bits(vg), bits(ve)), "pools differ"
    assert np.all(np.isfinite(out_g.float().cpu().numpy())), "non-finite output"
    del graph
    print("first-call capture ok", flush=True)


if __name__ == "__main__":
    main()
