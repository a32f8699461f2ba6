"""Upload a workload's inputs to the GPU as torch tensors (no attention arithmetic)."""

import numpy as np
import torch

from . import BF16


def to_device(arr, dtype, device):
    """Host numpy value (float32, or bf16 bit patterns) or tensor -> device tensor."""
    if isinstance(arr, torch.Tensor):
        return arr.to(device)
    a = np.ascontiguousarray(arr)
    if dtype == BF16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32)).to(device)


def int32_to_device(a, device):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a.astype(np.int32, copy=False)).to(device)


class DeviceInputs:
    """A workload's arrays on the GPU, in the library's layouts."""

    def __init__(self, case, device="cuda:0"):
        self.case = case
        self.device = device
        lay = case.layout
        self.q = to_device(case.q, case.dtype, device)
        self.k_pool = to_device(case.k_pool, case.dtype, device).contiguous()
        self.v_pool = to_device(case.v_pool, case.dtype, device).contiguous()
        self.k_new = to_device(case.k_new, case.dtype, device)
        self.v_new = to_device(case.v_new, case.dtype, device)
        self.table = int32_to_device(lay.table, device)
        self.slots = int32_to_device(lay.slot_mapping, device)
        self.seq_lens = int32_to_device(case.seq_lens, device)
        self.q_pos = int32_to_device(case.q_pos, device)
        self.cu = int32_to_device(case.cu_q_lens, device)
        self.q_pos_start = int32_to_device(lay.tail_pos, device)
        self.fill = None if lay.block_fill is None else torch.from_numpy(lay.block_fill).to(device)
