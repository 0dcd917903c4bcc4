"""Helpers for the GPU parity tests: device placement and case announcements."""
import numpy as np
import torch


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def case(msg: str) -> None:
    """Name the case before its GPU work starts, so a lost run still says what it was doing."""
    print(f"[case] {msg}", flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()
