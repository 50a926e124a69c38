"""GPU parity of the build-time design alternatives.

Each library in draft_kv_attention_amd.build.VARIANTS is the same sources built with
other macros (decode tiles in registers instead of the LDS pipeline, double-buffered
and non-temporal register tiles, three LDS stages, a separate decode combine kernel,
device-scope fences around the split ticket, the verifier's work-group-tiled kernel).
The binding is pointed at each library in turn and representative cases of the other
GPU test modules run through it against the fp64 oracle: the decode loop with slot
boundaries, the fused append step (fp32 tiny and bf16 3B layers), full-KV split plans
in bf16 and fp32, MASW == full-KV bitwise before the first slot, run-to-run
determinism, the verifier's row-block shapes and split plans, and the bf16 projection
with hidden slices.
"""
import os

import pytest
import torch

import draft_kv_attention_amd as M
from draft_kv_attention_amd import build as B
import tests.test_gpu_decode as TD
import tests.test_gpu_fused_verify as TV
import tests.test_gpu_materialize as TM

pytestmark = pytest.mark.gpu


@pytest.fixture(params=sorted(B.VARIANTS))
def variant(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    path = B.variant_path(request.param)
    if not os.path.exists(path):
        pytest.fail(f"{path} is not built: run python -m draft_kv_attention_amd.build")
    saved = (M._lib, M.LIB_PATH)
    M._lib, M.LIB_PATH = None, path
    try:
        assert M.lib()._name == path
        yield request.param
    finally:
        torch.cuda.synchronize()
        M._lib, M.LIB_PATH = saved


def test_variant_decode(variant):
    TD.test_tiny_decode_loop(3)
    TD.test_fullkv_decode_many_splits(16, 8, 128, torch.bfloat16)
    TD.test_fullkv_decode_many_splits(9, 3, 64, torch.float32)
    TD.test_masw_equals_fullkv_bitwise_before_first_slot(4)
    TD.test_determinism_bitwise()
    # fused append + attention against separate calls, fp32 tiny layer and bf16 3B layer
    TV.test_masw_decode_step_matches_separate_calls(TV.SI.TINY, 240, 3)
    TV.test_masw_decode_step_matches_separate_calls(TV.shape_of(TV.SI.DRAFT_3B, batch=2), 2300, 0)


def test_variant_verify(variant):
    TV.test_verify_ragged_small(32, 8, 6)
    TV.test_verify_ragged_small(64, 8, 8)
    TV.test_verify_split_plans(12, 64, 8)


def test_variant_projection(variant):
    TM.test_projection_hidden_splits_and_batch_groups(3072, 17)
