"""Oracle of the Ulysses layout permutes (TEST INFRASTRUCTURE ONLY: imported by tests/, bench.py's
CPU baseline and __graft_entry__.smoke, never by the library).

DeepSpeed Ulysses, one of the sequence-parallel methods the long-context recipe supports beside
Ring Attention (project page "How It Works"; Ring Attention summary, references), shards the
sequence over N devices and swaps that sharding for a head sharding around attention with an
all-to-all.  Device r holds x_r = X[:, r*Sl:(r+1)*Sl] (Sl = S/N rows, all H heads); after the
exchange device n holds all S rows of heads [n*H/N, (n+1)*H/N).  The device-local halves:
  pack:    send[n][b][s][j][d] = x[b][s][n*(H/N) + j][d]       (block n goes to device n)
  unpack:  x[b][s][n*(H/N) + j][d] = recv[n][b][s][j][d]       (block n came from device n)
written below as plain slice copies, plus the exchange itself for tests that emulate N devices.
"""
from __future__ import annotations

import numpy as np


def pack(x, n_devices: int):
    """x [B, Sl, H, D] -> send [N, B, Sl, H/N, D]: block n holds head group n of every local row."""
    b, sl, h, d = x.shape
    if h % n_devices:
        raise ValueError("heads must be a multiple of n_devices")
    hn = h // n_devices
    send = np.empty((n_devices, b, sl, hn, d), dtype=x.dtype)
    for n in range(n_devices):
        send[n] = x[:, :, n * hn:(n + 1) * hn, :]
    return send


def unpack(recv, n_devices: int):
    """recv [N, B, Sl, H/N, D] -> x [B, Sl, H, D]: block n supplies head group n."""
    n_, b, sl, hn, d = recv.shape
    if n_ != n_devices:
        raise ValueError("recv's first axis must be n_devices")
    x = np.empty((b, sl, hn * n_devices, d), dtype=recv.dtype)
    for n in range(n_devices):
        x[:, :, n * hn:(n + 1) * hn, :] = recv[n]
    return x


def alltoall(sends):
    """The exchange among N devices: device r receives block r of every device's send, in source
    order (recv_r[n] = send_n[r])."""
    n_devices = len(sends)
    return [np.stack([sends[n][r] for n in range(n_devices)]) for r in range(n_devices)]


def gather_sequence(recv):
    """[N, B, Sl, Hn, D] received blocks (source n = rows n*Sl...) -> [B, N*Sl, Hn, D]."""
    n_devices, b, sl, hn, d = recv.shape
    return np.concatenate([recv[n] for n in range(n_devices)], axis=1)
