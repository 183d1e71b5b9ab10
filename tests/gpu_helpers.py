"""Host <-> device plumbing for the GPU parity tests (numpy bit patterns in,
torch device tensors through the C ABI, numpy bit patterns out)."""
import sys

import numpy as np
import torch

import block_scaled_fp8_act_amd as fb


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU parity tests need a device")
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_to_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_codes_equal(got_q, got_s, want_q, want_s, what=""):
    got_q = np.asarray(got_q); want_q = np.asarray(want_q)
    if np.asarray(want_s).dtype == np.uint8:            # E8M0 scale bytes
        gs, ws = np.asarray(got_s, np.uint8), np.asarray(want_s, np.uint8)
    else:
        gs = np.asarray(got_s, np.float32).view(np.uint32)
        ws = np.asarray(want_s, np.float32).view(np.uint32)
    assert got_q.shape == want_q.shape and gs.shape == ws.shape, (got_q.shape, want_q.shape)
    bad_s = np.argwhere(gs != ws)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scales differ, first at {bad_s[:3].tolist()}: " \
        f"{gs[tuple(bad_s[0])]:#x} vs {ws[tuple(bad_s[0])]:#x}"
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[:3].tolist()}: " \
        f"{got_q[tuple(bad[0])]:#x} vs {want_q[tuple(bad[0])]:#x}"


def gpu_act_quant(x_bits):
    x = to_dev_bf16(x_bits)
    q, s = fb.act_quant_group(x)
    torch.cuda.synchronize()
    return host(q), host(s)


def gpu_weight_quant(w_bits):
    w = to_dev_bf16(w_bits)
    q, s = fb.weight_block_quant(w)
    torch.cuda.synchronize()
    return host(q), host(s)


def gpu_act_quant_ue8m0(x_bits):
    q, s = fb.act_quant_group(to_dev_bf16(x_bits), "ue8m0")
    torch.cuda.synchronize()
    return host(q), host(s)


def gpu_weight_quant_ue8m0(w_bits):
    q, s = fb.weight_block_quant(to_dev_bf16(w_bits), "ue8m0")
    torch.cuda.synchronize()
    return host(q), host(s)
