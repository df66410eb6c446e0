"""Seeded synthetic inputs for the chunk and decode workloads.

This module holds only the input recipes: random draws and the element-wise
recipe that turns them into the gate inputs. It computes nothing of the gated
delta rule itself, and it is the one module that both the CPU oracle's
callers and the HIP path's callers use, so that both see identical bf16/fp32
values.

Recipes (the workloads the chunk and decode kernels are measured on):
  q, k, v          ~ N(0, 1), stored bf16
  g  (log-decay)   = -exp(A_log) * softplus(a + dt_bias) in fp32, with
                     a ~ N(0, 1) per token and value head, A_log ~ U(0, ln 16)
                     per value head, dt_bias = 0
  beta             = sigmoid(N(0, 1)) in fp32
  h0               = 0.1 * N(0, 1) in fp32 (or absent)
  dO               ~ N(0, 1), stored bf16
  decode           q, k, v, a, b ~ N(0, 1) in bf16, A_log ~ U(0, ln 16) and
                   dt_bias = 0 in fp32 per value head, pool 0.1 * N(0, 1) fp32,
                   indices: a random permutation of 1..slots-1, the first
                   rows of it, with some rows set to 0 (the null block).
  short conv       x, dy ~ N(0, 1) bf16 [T, C]; weight ~ U(-1/sqrt(W), 1/sqrt(W))
                   bf16 [C, W] (the default init of a depthwise conv layer);
                   bias (when used) ~ U(-0.5, 0.5) bf16; carried states
                   ~ N(0, 1) bf16 [N or slots, C, W - 1]; pool indices as for
                   the decode step, 0 the null block.
  paged prefill    the chunk recipe without h0, a decode-style pool and
                   indices, and a has_initial_state mix of resumed (1) and
                   fresh (0) sequences.
Every draw comes from one CPU torch.Generator seeded explicitly.
"""
import math

import torch

K_DIM = 128
V_DIM = 128
BASE_SEED = 20260


def varlen_lengths(total, n, lo, hi, gen):
    """n log-uniform lengths in [lo, hi] rescaled to sum to ``total``.

    u ~ U(ln lo, ln hi), L = e^u, rescaled to the total and rounded half to
    even; the rounding remainder goes to the last sequence. If every length is
    then a multiple of 64, one token moves from the first to the second
    sequence so that the pack has ragged chunks.
    """
    u = torch.empty(n, dtype=torch.float64).uniform_(math.log(lo), math.log(hi), generator=gen)
    raw = torch.exp(u)
    scaled = raw * (total / raw.sum())
    lens = [int(x) for x in torch.round(scaled).tolist()]  # torch.round is half-to-even
    lens[-1] += total - sum(lens)
    if all(L % 64 == 0 for L in lens) and n >= 2:
        lens[0] -= 1
        lens[1] += 1
    return lens


def cu_from_lengths(lens):
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def chunk_inputs(lens, H, HV, seed, h0_std=0.1, with_do=False, K=K_DIM, V=V_DIM):
    """Inputs of one chunk call on a varlen pack with the given sequence lengths.

    Returns a dict of CPU tensors: q, k [T, H, K] bf16; v [T, HV, V] bf16;
    g, beta [T, HV] fp32; cu_seqlens [N+1] int32; h0 [N, HV, V, K] fp32 or None;
    do [T, HV, V] bf16 when ``with_do``.
    """
    gen = torch.Generator().manual_seed(seed)
    T = int(sum(lens))
    N = len(lens)
    q = torch.randn(T, H, K, generator=gen).to(torch.bfloat16)
    k = torch.randn(T, H, K, generator=gen).to(torch.bfloat16)
    v = torch.randn(T, HV, V, generator=gen).to(torch.bfloat16)
    a = torch.randn(T, HV, generator=gen, dtype=torch.float32)
    A_log = torch.empty(HV, dtype=torch.float32).uniform_(0.0, math.log(16.0), generator=gen)
    dt_bias = torch.zeros(HV, dtype=torch.float32)
    g = -torch.exp(A_log)[None, :] * torch.nn.functional.softplus(a + dt_bias[None, :])
    beta = torch.sigmoid(torch.randn(T, HV, generator=gen, dtype=torch.float32))
    h0 = None
    if h0_std is not None:
        h0 = h0_std * torch.randn(N, HV, V, K, generator=gen, dtype=torch.float32)
    out = dict(q=q, k=k, v=v, g=g.contiguous(), beta=beta, cu_seqlens=cu_from_lengths(lens), h0=h0)
    if with_do:
        out["do"] = torch.randn(T, HV, V, generator=gen).to(torch.bfloat16)
    return out


def decode_inputs(N, H, HV, slots, n_null, seed, K=K_DIM, V=V_DIM, pool=True):
    """Inputs of one decode step. Returns a dict of CPU tensors.

    q, k [N, H, K] bf16; v [N, HV, V] bf16; a, b [N, HV] bf16; A_log, dt_bias
    [HV] fp32; state_pool [slots, HV, V, K] fp32 (omitted with pool=False);
    ssm_state_indices [N] int32 drawn from a permutation of 1..slots-1 with
    ``n_null`` rows set to 0.
    """
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(N, H, K, generator=gen).to(torch.bfloat16)
    k = torch.randn(N, H, K, generator=gen).to(torch.bfloat16)
    v = torch.randn(N, HV, V, generator=gen).to(torch.bfloat16)
    a = torch.randn(N, HV, generator=gen).to(torch.bfloat16)
    b = torch.randn(N, HV, generator=gen).to(torch.bfloat16)
    A_log = torch.empty(HV, dtype=torch.float32).uniform_(0.0, math.log(16.0), generator=gen)
    dt_bias = torch.zeros(HV, dtype=torch.float32)
    perm = torch.randperm(slots - 1, generator=gen)[:N] + 1
    null_rows = torch.randperm(N, generator=gen)[:n_null]
    idx = perm.clone()
    idx[null_rows] = 0
    out = dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias,
               ssm_state_indices=idx.to(torch.int32))
    if pool:
        out["state_pool"] = 0.1 * torch.randn(slots, HV, V, K, generator=gen, dtype=torch.float32)
    return out


def paged_inputs(lens, H, HV, slots, n_null, n_fresh, seed, K=K_DIM, V=V_DIM):
    """Inputs of one paged chunk call: those of ``chunk_inputs`` (without h0)
    plus state_pool [slots, HV, V, K] fp32 = 0.1 * N(0, 1), ssm_state_indices
    [N] int32 (the first N entries of a random permutation of 1..slots-1, with
    ``n_null`` random rows set to 0, the null block) and has_initial_state [N]
    int32 (1, with ``n_fresh`` random rows set to 0: fresh prompts).
    """
    out = chunk_inputs(lens, H, HV, seed, h0_std=None, K=K, V=V)
    gen = torch.Generator().manual_seed(seed + 500)
    N = len(lens)
    idx = torch.randperm(slots - 1, generator=gen)[:N] + 1
    idx[torch.randperm(N, generator=gen)[:n_null]] = 0
    init = torch.ones(N, dtype=torch.int32)
    init[torch.randperm(N, generator=gen)[:n_fresh]] = 0
    out.update(state_pool=0.1 * torch.randn(slots, HV, V, K, generator=gen, dtype=torch.float32),
               ssm_state_indices=idx.to(torch.int32), has_initial_state=init)
    return out


def conv_inputs(lens, C, W, seed, bias=False, state=False, with_dy=False):
    """Inputs of one short-convolution call on a varlen pack. Returns a dict of
    CPU tensors: x [T, C] bf16, weight [C, W] bf16, bias [C] bf16 or None,
    cu_seqlens [N+1] int32, state_in [N, C, W-1] bf16 or None, dy [T, C] bf16
    when ``with_dy``."""
    gen = torch.Generator().manual_seed(seed)
    T, N = int(sum(lens)), len(lens)
    bound = 1.0 / math.sqrt(W)
    out = dict(
        x=torch.randn(T, C, generator=gen).to(torch.bfloat16),
        weight=torch.empty(C, W).uniform_(-bound, bound, generator=gen).to(torch.bfloat16),
        bias=torch.empty(C).uniform_(-0.5, 0.5, generator=gen).to(torch.bfloat16) if bias else None,
        cu_seqlens=cu_from_lengths(lens),
        state_in=torch.randn(N, C, W - 1, generator=gen).to(torch.bfloat16) if state else None,
    )
    if with_dy:
        out["dy"] = torch.randn(T, C, generator=gen).to(torch.bfloat16)
    return out


def conv_pool_inputs(N, C, W, slots, n_null, seed):
    """A conv state pool [slots, C, W-1] bf16 ~ N(0, 1) and indices [N] int32:
    the first N entries of a random permutation of 1..slots-1 with ``n_null``
    random rows set to 0 (the null block)."""
    gen = torch.Generator().manual_seed(seed)
    pool = torch.randn(slots, C, W - 1, generator=gen).to(torch.bfloat16)
    idx = torch.randperm(slots - 1, generator=gen)[:N] + 1
    idx[torch.randperm(N, generator=gen)[:n_null]] = 0
    return pool, idx.to(torch.int32)


# The workloads, by name. Sizes as measured and parity-tested.
WORKLOADS = {
    "fwd_1x256_h1": dict(kind="fwd", lens=[256], H=1, HV=1, h0_std=None, seed=BASE_SEED + 0),
    "fwd_4x4096_h16_hv32": dict(kind="fwd", lens=[4096] * 4, H=16, HV=32, h0_std=0.1,
                                seed=BASE_SEED + 1),
    "fwd_varlen12_32768_h16_hv32": dict(kind="fwd", lens=None, total=32768, nseq=12, H=16,
                                        HV=32, h0_std=None, seed=BASE_SEED + 2),
    "fwdbwd_2x8192_h16_hv32": dict(kind="fwdbwd", lens=[8192] * 2, H=16, HV=32, h0_std=0.1,
                                   seed=BASE_SEED + 3),
    "decode_256_pool512_h16_hv32": dict(kind="decode", N=256, H=16, HV=32, slots=512, n_null=16,
                                        seed=BASE_SEED + 4),
    "paged_8x512_h8_hv16_pool64": dict(kind="paged", lens=[512] * 8, H=8, HV=16, slots=64,
                                       n_null=0, n_fresh=4, seed=BASE_SEED + 5),
    # one long sequence (the long-context rows of the Cake page's tests)
    # many short sequences: the pages' 32 x 512 and 128 x 128 packs of 16384 tokens
    "fwdbwd_32x512_h16_hv32": dict(kind="fwdbwd", lens=[512] * 32, H=16, HV=32, h0_std=0.1,
                                   seed=BASE_SEED + 13),
    "fwdbwd_128x128_h16_hv32": dict(kind="fwdbwd", lens=[128] * 128, H=16, HV=32, h0_std=0.1,
                                    seed=BASE_SEED + 14),
    "fwdbwd_1x65536_h16_hv32": dict(kind="fwdbwd", lens=[65536], H=16, HV=32, h0_std=0.1,
                                    seed=BASE_SEED + 11),
    "fwdbwd_1x131072_h16_hv32": dict(kind="fwdbwd", lens=[131072], H=16, HV=32, h0_std=0.1,
                                     seed=BASE_SEED + 12),
    # one GPU's share of the head-sharded layer at TP = 2 (8 key / 16 value heads)
    "fwd_4x4096_h8_hv16": dict(kind="fwd", lens=[4096] * 4, H=8, HV=16, h0_std=0.1,
                               seed=BASE_SEED + 21),
    "fwd_varlen12_32768_h8_hv16": dict(kind="fwd", lens=None, total=32768, nseq=12, H=8, HV=16,
                                       h0_std=None, seed=BASE_SEED + 22, lens_from=BASE_SEED + 2),
    "fwdbwd_2x8192_h8_hv16": dict(kind="fwdbwd", lens=[8192] * 2, H=8, HV=16, h0_std=0.1,
                                  seed=BASE_SEED + 23),
    # the short convolution over the q, k, v channels of the fwd+bwd pack
    # (2 x 128 x 16 key-head channels + 128 x 32 value-head channels), width 4
    "conv_2x8192_c8192_w4": dict(kind="conv", lens=[8192] * 2, C=8192, W=4, seed=BASE_SEED + 6),
}


def workload_lengths(name):
    w = WORKLOADS[name]
    if w.get("lens") is not None:
        return list(w["lens"])
    # (the TP = 2 share of the varlen pack keeps the full pack's lengths)
    gen = torch.Generator().manual_seed(w.get("lens_from", w["seed"]) + 1000)
    return varlen_lengths(w["total"], w["nseq"], 256, 8192, gen)


def workload_inputs(name):
    w = WORKLOADS[name]
    if w["kind"] == "decode":
        return decode_inputs(w["N"], w["H"], w["HV"], w["slots"], w["n_null"], w["seed"])
    if w["kind"] == "conv":
        return conv_inputs(w["lens"], w["C"], w["W"], w["seed"], with_dy=True)
    if w["kind"] == "paged":
        return paged_inputs(workload_lengths(name), w["H"], w["HV"], w["slots"], w["n_null"],
                            w["n_fresh"], w["seed"])
    return chunk_inputs(workload_lengths(name), w["H"], w["HV"], w["seed"], h0_std=w["h0_std"],
                        with_do=(w["kind"] == "fwdbwd"))
