"""GPU check of fp8_quantize_noalloc, the quantize entry point that allocates
nothing (its per-tensor scratch is a static device array of the library).

Called through the C ABI, it must give bit for bit what fp8_quantize (with a
caller workspace) gives, on two calls in a row, the second with a smaller
input: the scratch keeps the first call's partial maxima, and the second
call must not read them."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from gpu_helpers import dev, host, say

pytestmark = pytest.mark.gpu


def _input(rows, cols, seed, scale):
    rng = np.random.default_rng(seed)
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = workloads.draw_x(wl, rows, cols, rng) * np.float32(scale)
    return dev(workloads.f32_to_bf16_bits(x))


@pytest.mark.parametrize("gran", [fb.GRAN_TENSOR, fb.GRAN_TILE_1x128, fb.GRAN_ROW])
@pytest.mark.parametrize("fmt", [fb.E4M3, fb.E5M2])
def test_noalloc_quantize_matches_workspace_entry_point(gran, fmt):
    lib = fb.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    # the first call is large (3584 partial maxima for a per-tensor scale) with
    # a large amax, the second small (8 partials) with a 1000x smaller one: the
    # first call's partial maxima, left in the scratch, would raise the second
    # call's amax and scale if it read them
    for call, (rows, cols, scale) in enumerate([(4096, 7168, 1000.0), (128, 512, 1.0)]):
        label = f"noalloc quantize call {call} gran={gran} fmt={fmt} {rows}x{cols}"
        say(label)
        x = _input(rows, cols, 90 + call, scale)
        q_ref, s_ref = fb.fp8_quantize(x, fmt, gran)
        q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
        s = torch.empty(fb.scale_shape(gran, rows, cols), dtype=torch.float32, device="cuda")
        st = lib.fp8_quantize_noalloc(x.data_ptr(), fb.DT_BF16, rows, cols, fmt, gran, q.data_ptr(), s.data_ptr(),
                                      stream)
        assert st == 0, fb.fp8_status_string(st)
        torch.cuda.synchronize()
        assert np.array_equal(host(q), host(q_ref)), label + ": codes differ"
        assert np.array_equal(host(s).view(np.uint32), host(s_ref).view(np.uint32)), label + ": scales differ"


def test_noalloc_quantize_host_errors_and_empty():
    lib = fb.load_library()
    one = torch.empty(1, dtype=torch.float32, device="cuda")
    q = torch.empty((16, 128), dtype=torch.uint8, device="cuda")
    x = torch.zeros((16, 128), dtype=torch.bfloat16, device="cuda")
    # bad enum, bad shape, missing pointers: rejected before any launch
    assert lib.fp8_quantize_noalloc(x.data_ptr(), 5, 16, 128, 0, 0, q.data_ptr(), one.data_ptr(), None) == 2
    assert lib.fp8_quantize_noalloc(x.data_ptr(), 1, 16, 100, 0, 0, q.data_ptr(), one.data_ptr(), None) == 3
    assert lib.fp8_quantize_noalloc(None, 1, 16, 128, 0, 0, q.data_ptr(), one.data_ptr(), None) == 1
    # an empty per-tensor call writes the scale 1.0 only
    one.fill_(7.0)
    assert lib.fp8_quantize_noalloc(x.data_ptr(), 1, 0, 128, 0, 0, q.data_ptr(), one.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert float(one.item()) == 1.0
