"""Parity at the largest sizes each kernel family takes, and just past them (where the
host picks the next family), against the oracle through the C ABI.  Which kernels run
follows from the selection rules of the library (the sizes are chosen against them):
  - small-batch routing (router logits, then top-k + grouping in one block): T <= 4 (the
    layer's own limits, E <= 2048 and k <= 64, keep T k <= 256);
  - the single-launch few-token MXFP4 forward: T <= 16 with every expert's token rows in
    its LDS stage (at most 48 KB: H, I small enough for 16 rows);
  - the RVQ3 table lookups: T <= 64, the codeword table, codebooks and token slices within
    the LDS of one block (H up to 4864 here);
  - the grouped GEMMs: T k >= 8 E (experts average at least 8 tokens)."""
import pytest

import moe_synth as syn
from cases import host_case
from test_gpu_parity import run_small

pytestmark = pytest.mark.gpu

TINY = syn.WORKLOADS["tiny"]
RVQ = syn.WORKLOADS["rvq16"]


def test_small_batch_routing_at_its_largest():
    # T k = 256 slots over E = 2048 experts (64 logits a lane): the single-block top-k and
    # grouping at their limits
    w = syn.shrink(TINY, T=4, H=256, I=128, E=2048, k=64, x_dtype="bf16", with_dy=True, x_key=90)
    run_small(host_case(w), name="route-small-max")


def test_routing_past_the_small_batch_limit():
    # T = 5 at the layer's largest E and k: the per-token top-k launch (64 logits a lane,
    # 64 ranks) and the separate grouping launch
    w = syn.shrink(TINY, T=5, H=256, I=128, E=2048, k=64, x_dtype="bf16", with_dy=True, x_key=91)
    run_small(host_case(w), name="route-past-small")


def test_single_launch_decode_at_sixteen_tokens():
    # 16 tokens (the few-token limit), 64 units, h planes unpacked (more than 8 tokens)
    w = syn.shrink(TINY, T=16, H=1024, I=512, E=64, k=8, x_dtype="bf16", with_dy=True, x_key=92)
    run_small(host_case(w), name="dec-fused-T16")


def test_seventeen_tokens_leave_the_few_token_path():
    w = syn.shrink(TINY, T=17, H=1024, I=512, E=64, k=8, x_dtype="bf16", with_dy=True, x_key=93)
    run_small(host_case(w), name="dec-past-T16")


@pytest.mark.parametrize("T", [64, 65])
def test_rvq3_table_lookups_at_sixty_four_tokens_and_past(T):
    # T = 64: the table-lookup kernels at their token limit; T = 65: the generic RVQ3 kernels
    w = syn.shrink(RVQ, T=T, H=1024, I=1024, E=64, k=4, with_dy=True, x_key=94)
    run_small(host_case(w), name=f"rvq3-T{T}")


def test_rvq3_table_lookups_at_the_widest_row():
    # H = 4864: 608 vectors a row (four phase classes, a three-quarter last window); the
    # gate/up block's table, codebooks and two token slices fill 159 KB of LDS
    w = syn.shrink(RVQ, T=4, H=4864, I=512, E=8, k=2, with_dy=True, x_key=95)
    run_small(host_case(w), name="rvq3-wide-H")


@pytest.mark.parametrize("T", [64, 63])
def test_grouped_gemm_threshold(T):
    # T k = 8 E exactly (grouped GEMMs) and one token fewer (the generic kernels)
    w = syn.shrink(TINY, T=T, H=512, I=512, E=16, k=2, x_dtype="bf16", with_dy=True, x_key=96)
    run_small(host_case(w), name=f"mm-threshold-T{T}")
