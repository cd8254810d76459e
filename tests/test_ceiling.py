"""libceiling.so, the benchmark's measurement helpers (include/lcsi_ceiling.h).

Host side (no GPU): the library exports every function the header declares
and refuses bad arguments before launching anything.  GPU: the MFMA loop
computes the products it claims (each wave's output is the sum of all its
accumulators, which has a closed form on the CPU), the streaming read
touches every 16-byte unit exactly once (its XOR per thread, checked on the
CPU), and the gather lands every listed row's chunks where the read-back
expects them (clamped row numbers included)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcsi_ceiling.h")
LIB = os.path.join(ROOT, "long_context_sparse_idx_amd", "libceiling.so")
FAKE = 0x7F0000000000  # aligned, never dereferenced


def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB)
    L.lcsi_ceiling_data_elems.restype = ctypes.c_size_t
    L.lcsi_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    L.lcsi_ceiling_mfma.restype = ctypes.c_int
    L.lcsi_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    L.lcsi_ceiling_read.restype = ctypes.c_int
    L.lcsi_ceiling_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.lcsi_ceiling_gather.restype = ctypes.c_int
    return L


def test_exports_every_declared_function():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = set(re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}()]*\)\s*;", text))
    assert names == {"lcsi_ceiling_data_elems", "lcsi_ceiling_mfma", "lcsi_ceiling_read", "lcsi_ceiling_gather"}
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert names <= exported


def test_bad_arguments_are_refused_before_launch():
    L = lib()
    # (every call fails its checks, so nothing is dereferenced or launched)
    assert L.lcsi_ceiling_mfma(None, ctypes.c_void_p(FAKE), 1, 4, 0, None) == -1
    assert L.lcsi_ceiling_mfma(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 0, 4, 0, None) == -1
    assert L.lcsi_ceiling_mfma(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1, 6, 0, None) == -1  # blocks % 4
    assert L.lcsi_ceiling_mfma(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1, 4, 2, None) == -1  # mode
    assert L.lcsi_ceiling_mfma(ctypes.c_void_p(FAKE + 2), ctypes.c_void_p(FAKE), 1, 4, 0, None) == -5
    assert L.lcsi_ceiling_read(None, 16, ctypes.c_void_p(FAKE), 1, None) == -1
    assert L.lcsi_ceiling_read(ctypes.c_void_p(FAKE), 24, ctypes.c_void_p(FAKE), 1, None) == -1  # not 16-B units
    assert L.lcsi_ceiling_read(ctypes.c_void_p(FAKE), 16, ctypes.c_void_p(FAKE), 0, None) == -1
    assert L.lcsi_ceiling_read(ctypes.c_void_p(FAKE + 4), 16, ctypes.c_void_p(FAKE), 1, None) == -5
    assert L.lcsi_ceiling_read(ctypes.c_void_p(FAKE), 16, ctypes.c_void_p(FAKE + 2), 1, None) == -5
    G = L.lcsi_ceiling_gather
    F = ctypes.c_void_p(FAKE)
    assert G(None, 10, 1152, F, 1, 1, F, None) == -1
    assert G(F, 0, 1152, F, 1, 1, F, None) == -1            # no rows
    assert G(F, 10, 1160, F, 1, 1, F, None) == -1           # row longer than 1152 bytes
    assert G(F, 10, 24, F, 1, 1, F, None) == -1             # not whole 16-byte chunks
    assert G(F, 10, 1152, F, 1, 65, F, None) == -1          # more than 64 lists
    assert G(F, 10, 1152, F, 0, 1, F, None) == -1
    assert G(ctypes.c_void_p(FAKE + 8), 10, 1152, F, 1, 1, F, None) == -5
    assert G(F, 10, 1152, ctypes.c_void_p(FAKE + 2), 1, 1, F, None) == -5


NWAVE, ROWS, DIM = 8, 64, 128   # waves per workgroup, query rows per wave, dims


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1])
def test_mfma_loop_computes_its_products(mode):
    """Wave w of workgroup b multiplies its 64 query rows (data rows
    ((b % 64) * 8 + w) * 64 ..) by key blocks of 32 rows: mode 0 the four
    blocks of keys 0..127, `blocks / 4` times; mode 1 block it % 8 of keys
    0..255 at step it.  The sum of all accumulators of a wave is therefore
    (sum of its query rows) . (sum of the key rows it met, with multiplicity).
    Positive operands, so the fp32 sums have no cancellation."""
    L = lib()
    n = L.lcsi_ceiling_data_elems()
    nq = 64 * NWAVE * ROWS
    assert n == nq * DIM + 256 * DIM
    g = torch.Generator().manual_seed(7 + mode)
    host = (torch.rand(n, generator=g) / 8).to(torch.bfloat16)
    data = host.cuda()
    n_wg, blocks = 70, 16       # (70 > 64: workgroups 64.. reuse query rows, as the kernel wraps)
    out = torch.full((n_wg * NWAVE,), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.lcsi_ceiling_mfma(ctypes.c_void_p(data.data_ptr()), ctypes.c_void_p(out.data_ptr()), n_wg, blocks,
                             mode, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    x = host.float().double().numpy()
    q = x[:nq * DIM].reshape(64 * NWAVE, ROWS, DIM)
    k = x[nq * DIM:].reshape(256, DIM)
    if mode == 0:
        ksum = (blocks // 4) * k[:128].sum(axis=0)
    else:
        ksum = np.zeros(DIM)
        for it in range(blocks):
            cb = it % 8
            ksum += k[cb * 32:(cb + 1) * 32].sum(axis=0)
    got = out.cpu().double().numpy().reshape(n_wg, NWAVE)
    for b in range(n_wg):
        for w in range(NWAVE):
            want = q[(b % 64) * NWAVE + w].sum(axis=0) @ ksum
            assert abs(got[b, w] - want) <= 1e-3 * want, (b, w, got[b, w], want)


@pytest.mark.gpu
def test_streaming_read_touches_every_unit_once():
    """Thread t (of n_wg * 256) XORs the four words of units t, t + S, ...
    (S = n_wg * 256); the buffer's length is not a multiple of the loop's
    eight-unit stride, so the tail loop is covered too."""
    L = lib()
    n_wg = 3
    S = n_wg * 256
    units = 8 * S * 5 + 37
    g = torch.Generator().manual_seed(11)
    host = torch.randint(0, 2 ** 31 - 1, (units * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.cuda()
    out = torch.zeros(S, dtype=torch.int32, device="cuda")
    rc = L.lcsi_ceiling_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(units * 16),
                             ctypes.c_void_p(out.data_ptr()), n_wg,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    w = host.numpy().view(np.uint32).reshape(units, 4)
    per_unit = w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    want = np.zeros(S, np.uint32)
    for t in range(S):
        want[t] = np.bitwise_xor.reduce(per_unit[t::S])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)


@pytest.mark.gpu
@pytest.mark.parametrize("row_bytes,tiles", [(1152, 5), (256, 2)])
def test_gather_lands_every_listed_row(row_bytes, tiles):
    """Thread i of workgroup w XORs LDS unit i of each of its lists: chunk
    i % cpr of list entry i // cpr (cpr = row_bytes / 16), i.e. 16 bytes of
    row idx[w, t, i // cpr] (clamped to the rows present).  Some row numbers
    are out of range on purpose: -3 and n_rows + 5 read rows 0 and n_rows - 1."""
    L = lib()
    n_rows, n_wg = 700, 6
    g = torch.Generator().manual_seed(13)
    host = torch.randint(0, 2 ** 31 - 1, (n_rows * row_bytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    idx = torch.randint(0, n_rows, (n_wg, tiles, 32), generator=g, dtype=torch.int64).to(torch.int32)
    idx[0, 0, 0], idx[1, tiles - 1, 3] = -3, n_rows + 5
    rows, didx = host.cuda(), idx.cuda()
    out = torch.zeros(n_wg * 256, dtype=torch.int32, device="cuda")
    rc = L.lcsi_ceiling_gather(ctypes.c_void_p(rows.data_ptr()), n_rows, row_bytes, ctypes.c_void_p(didx.data_ptr()),
                               n_wg, tiles, ctypes.c_void_p(out.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32).reshape(n_rows, row_bytes // 16, 4)
    unit = words[:, :, 0] ^ words[:, :, 1] ^ words[:, :, 2] ^ words[:, :, 3]
    cpr = row_bytes // 16
    cl = np.clip(idx.numpy(), 0, n_rows - 1)
    want = np.zeros((n_wg, 256), np.uint32)
    for w in range(n_wg):
        for t in range(tiles):
            for i in range(256):
                want[w, i] ^= unit[cl[w, t, i // cpr], i % cpr]
    assert np.array_equal(out.cpu().numpy().view(np.uint32).reshape(n_wg, 256), want)
