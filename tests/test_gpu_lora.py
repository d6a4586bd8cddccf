"""GPU parity of the shared low-rank adapter (LazyLoRA README, "LoRA"): forward, input
gradient and adapter gradients through every expert kernel family, against the fp64 oracle
on the same seeded inputs (max|err| / max|ref| <= 1e-4; routing bit-exact)."""
import pytest

import moe_synth as syn
from cases import act_tensor, device_layer, host_case, lora_parity

pytestmark = pytest.mark.gpu

TINY = syn.WORKLOADS["tiny"]
SCALE = 2.0  # alpha / r = 32 / 16, the README's rank and alpha


def run_lora(c, name, flags=0, rank=16, saved=(True, False)):
    from quantized_moe_route_amd import _lib as C
    L = device_layer(c, max_tokens=max(c.w.T, 1), flags=flags | C.MOE_F_LORA)
    lora_parity(c, L, name, rank=rank, scale=SCALE, saved=saved)
    L.close()


def _case(w, act=0):
    c = host_case(w, with_dy=True)
    c.act = act
    return c


def test_lora_tiny_generic_fp32_tokens():
    run_lora(_case(syn.shrink(TINY, with_dy=True)), "lora-tiny")


def test_lora_bias_situ_generic_bf16():
    run_lora(_case(syn.shrink(TINY, x_dtype="bf16", bias_sd=0.5, with_dy=True, x_key=50), act=1), "lora-situ-bias")


def test_lora_single_token_decode_kernels():
    # one token, bf16, H and I multiples of 256: the few-token stream kernels
    run_lora(_case(syn.shrink(TINY, T=1, H=1024, I=512, E=16, k=8, x_dtype="bf16", with_dy=True, x_key=51)),
             "lora-dec-T1", rank=8)


def test_lora_few_tokens_decode_kernels():
    run_lora(_case(syn.shrink(TINY, T=5, H=512, I=768, E=12, k=3, x_dtype="bf16", with_dy=True, x_key=52)),
             "lora-dec-few")


@pytest.mark.parametrize("rank", [1, 6])
def test_lora_fused_decode_odd_ranks_situ(rank):
    # the single few-token launch forms the adapter's gate/up and down terms itself: ranks
    # that are not a multiple of four (scalar rank sums), SiTU, a router bias, three tokens
    run_lora(_case(syn.shrink(TINY, T=3, H=768, I=512, E=10, k=4, x_dtype="bf16", bias_sd=0.5, with_dy=True,
                              x_key=59 + rank), act=1), f"lora-fused-rank{rank}", rank=rank)


def test_lora_grouped_gemm_paths():
    # T k >= 8 E with H, I multiples of 512: grouped-GEMM forward and backward (dg/du as bf16
    # hi + lo planes); rank 32 takes the square GEMM tiles
    run_lora(_case(syn.shrink(TINY, T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16", with_dy=True, x_key=53)),
             "lora-mm", rank=32)


def test_lora_block_scaled_gateup():
    from quantized_moe_route_amd import _lib as C
    run_lora(_case(syn.shrink(TINY, T=300, H=1024, I=512, E=16, k=3, x_dtype="bf16", with_dy=True, x_key=54)),
             "lora-mx", flags=C.MOE_F_MX_GATEUP)


def test_lora_rvq3_paths():
    run_lora(_case(syn.shrink(syn.WORKLOADS["rvq16"], T=10, H=512, I=768, E=12, k=3, with_dy=True, x_key=55)),
             "lora-rvq3-gather")
    run_lora(_case(syn.shrink(syn.WORKLOADS["rvq16"], T=24, H=256, I=128, E=12, k=3, with_dy=True, x_key=56), act=1),
             "lora-rvq3-generic-situ", rank=4)
    # ~13 tokens per expert with an adapter: the codeword-gather kernels in four passes of up
    # to 4 tokens, the weights re-read per pass
    run_lora(_case(syn.shrink(syn.WORKLOADS["rvq16"], T=40, H=256, I=512, E=6, k=2, with_dy=True, x_key=57)),
             "lora-rvq3-gather-passes")


def test_lora_zero_tokens_gives_zero_gradients():
    import torch

    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, with_dy=True)
    c = host_case(w, with_dy=True)
    A, B = syn.lora_adapter(w, 16)
    L = device_layer(c, max_tokens=8, flags=C.MOE_F_LORA)
    L.set_lora([q.to_device(a) for a in A], [q.to_device(b) for b in B], SCALE)
    x = act_tensor(c.x[:0], w.x_dtype)
    r = L.new_routing(0)
    dx, dA, dB = L.backward_lora(x, x, r)
    torch.cuda.synchronize()
    assert all(float(t.abs().max()) == 0.0 for t in dA + dB)
    L.close()


@pytest.mark.parametrize("T,rank", [(100, 48), (5, 64)])
def test_lora_ranks_above_32(T, rank):
    # ranks past 32 split the row sums and the wide products into two passes over the rank;
    # 100 tokens take the tall products, 5 the per-output dot products
    run_lora(_case(syn.shrink(TINY, T=T, H=512, I=256, E=8, k=4, x_dtype="bf16", with_dy=True, x_key=58 + T)),
             f"lora-rank{rank}", rank=rank)
