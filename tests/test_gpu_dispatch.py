"""Dispatch counts of the entry points.

Each call is captured into a HIP graph through the runtime's own graph API (the
copy of libamdhip64 that torch and libdsaidx share), and the graph's nodes are
counted.  The fused entry is one kernel dispatch for the whole call: turning
the separate rope, quantisation, gate-fold and cache-write launches into one
is the point of the method ([sglang-fuse] section Benchmark; [vllm-47335]
Kernel-level evidence).  The query-only and key entries are one dispatch
each; top-k is one for rows of up to 32768 logits and four beyond.  No node
is a memset or a copy: the library enqueues kernels only."""
import ctypes

import pytest
import torch

import rope_fp8_quant_amd as R
from rope_fp8_quant_amd import workloads as W
from gpu_util import DeviceCase

pytestmark = pytest.mark.gpu

KERNEL_NODE = 0                  # hipGraphNodeTypeKernel
CAPTURE_THREAD_LOCAL = 1         # hipStreamCaptureModeThreadLocal


@pytest.fixture(scope="module")
def hip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()
    R.lib()
    paths = sorted({line.split()[-1] for line in open("/proc/self/maps")
                    if "libamdhip64" in line and line.split()[-1].startswith("/")})
    assert len(paths) == 1, paths    # one HIP runtime in the process
    h = ctypes.CDLL(paths[0])
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    h.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
    h.hipStreamEndCapture.argtypes = [vp, ctypes.POINTER(vp)]
    h.hipGraphGetNodes.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(sz)]
    h.hipGraphNodeGetType.argtypes = [vp, ctypes.POINTER(ctypes.c_int)]
    h.hipGraphDestroy.argtypes = [vp]
    for f in ("hipStreamBeginCapture", "hipStreamEndCapture", "hipGraphGetNodes",
              "hipGraphNodeGetType", "hipGraphDestroy"):
        getattr(h, f).restype = ctypes.c_int
    return h


def node_types(hip, call):
    """Types of the graph nodes that `call(stream)` enqueues."""
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    handle = ctypes.c_void_p(s.cuda_stream)
    assert hip.hipStreamBeginCapture(handle, CAPTURE_THREAD_LOCAL) == 0
    graph = ctypes.c_void_p()
    try:
        call(s)
    finally:
        rc = hip.hipStreamEndCapture(handle, ctypes.byref(graph))
    assert rc == 0
    try:
        n = ctypes.c_size_t(0)
        assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
        nodes = (ctypes.c_void_p * max(n.value, 1))()
        assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
        types = []
        for i in range(n.value):
            t = ctypes.c_int(-1)
            assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
            types.append(t.value)
        return types
    finally:
        hip.hipGraphDestroy(graph)


@pytest.mark.parametrize("T", [64, 3000])
def test_prep_entry_dispatch_counts(hip, T):
    wl = W.make(T, 64, seed=5)
    c = DeviceCase(wl)
    qa, ka, rope = c.qa(), c.ka(), c.rope()
    assert node_types(hip, lambda s: R.dsaidx_qk_fused(qa, ka, rope, stream=s)) == [KERNEL_NODE]
    assert node_types(hip, lambda s: R.dsaidx_q_rope_quant_fold(qa, rope, stream=s)) == [KERNEL_NODE]
    assert node_types(hip, lambda s: R.dsaidx_k_norm_rope_quant_store(ka, rope, stream=s)) == [KERNEL_NODE]
    assert node_types(hip, lambda s: R.dsaidx_k_only_prepare_store(ka, rope, stream=s)) == [KERNEL_NODE]

    def q_then_k(s):
        R.dsaidx_q_rope_quant_fold(qa, rope, stream=s)
        R.dsaidx_k_norm_rope_quant_store(ka, rope, stream=s)
    assert node_types(hip, q_then_k) == [KERNEL_NODE, KERNEL_NODE]


def test_empty_call_enqueues_nothing(hip):
    wl = W.make(8, 64, seed=6)
    c = DeviceCase(wl)
    qa, ka, rope = c.qa(), c.ka(), c.rope()
    qa.num_tokens = 0
    ka.num_tokens = 0
    assert node_types(hip, lambda s: R.dsaidx_qk_fused(qa, ka, rope, stream=s)) == []


@pytest.mark.parametrize("cols,dispatches", [(16384, 1), (32768, 1), (32769, 4), (131072, 4)])
def test_topk_dispatch_counts(hip, cols, dispatches):
    rows, k = 8, 2048
    stride = cols + (-cols) % 4                      # rows start 16-byte aligned
    logits = torch.randn((rows, stride), dtype=torch.float32, device="cuda")[:, :cols]
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    need = R.dsaidx_topk_workspace_bytes(rows, cols, k)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    types = node_types(hip, lambda s: R.dsaidx_topk_per_row(logits, k, out, stream=s, workspace=ws))
    assert types == [KERNEL_NODE] * dispatches
