"""Oracle for Tensor Fusion: the buffer plan, pack and unpack.

Test infrastructure: only the test suite, the package smoke check and the
bench's cpu_baseline leg use the oracle; the product path never does.

Source: "Horovod: Fast and Easy Distributed Deep Learning in TensorFlow"
(paper summary page), section 3.4, "Tensor Fusion" steps 1-6: pick the
first ready tensors that fit in the remaining buffer space and share a data
type, copy them contiguously into the fusion buffer (64 MB by default),
reduce the buffer once, copy the results back out, repeat.

Readings where the page is silent:
* ready order is the order the caller lists the tensors in (the page: the
  last layer's gradients are ready first); the plan never reorders;
* a buffer is closed at the first tensor that does not fit or changes the
  data type (no skipping ahead to a later, smaller tensor);
* an exact fit counts as a fit;
* a tensor larger than the whole buffer is reduced alone, in a buffer of
  its own;
* tensors are concatenated densely, without padding.
"""
from typing import List, Sequence, Tuple

import numpy as np

ELEM_BYTES = {0: 4, 1: 2}  # F32, BF16


def fuse_plan(n_elems: Sequence[int], dtypes: Sequence[int], cap_bytes: int
              ) -> Tuple[List[int], List[int], List[int], List[int]]:
    """Return (buf_of, off_of, fill, buf_dtype).

    buf_of[t]  - buffer id of tensor t
    off_of[t]  - element offset of tensor t inside its buffer
    fill[k]    - number of elements in buffer k
    buf_dtype  - data type of buffer k
    """
    buf_of, off_of, fill, buf_dtype = [], [], [], []
    cur = -1            # index of the open buffer, -1 if none
    cur_bytes = 0
    for n, dt in zip(n_elems, dtypes):
        nbytes = int(n) * ELEM_BYTES[int(dt)]
        if nbytes > cap_bytes:
            # oversize: a buffer of its own, and the open buffer is closed
            fill.append(int(n))
            buf_dtype.append(int(dt))
            buf_of.append(len(fill) - 1)
            off_of.append(0)
            cur = -1
            cur_bytes = 0
            continue
        fits = cur >= 0 and buf_dtype[cur] == int(dt) and cur_bytes + nbytes <= cap_bytes
        if not fits:
            fill.append(0)
            buf_dtype.append(int(dt))
            cur = len(fill) - 1
            cur_bytes = 0
        buf_of.append(cur)
        off_of.append(fill[cur])
        fill[cur] += int(n)
        cur_bytes += nbytes
    return buf_of, off_of, fill, buf_dtype


def fuse_pack(tensors: Sequence[np.ndarray], buf_of, off_of, fill, dtype) -> List[np.ndarray]:
    """Step 3: copy every tensor of one worker into its fusion buffer."""
    bufs = [np.zeros(int(f), dtype=dtype) for f in fill]
    for t, x in enumerate(tensors):
        o = int(off_of[t])
        bufs[buf_of[t]][o:o + x.size] = x.reshape(-1)
    return bufs


def fuse_unpack(bufs: Sequence[np.ndarray], buf_of, off_of, sizes) -> List[np.ndarray]:
    """Step 5: copy every tensor's slice back out of its fusion buffer."""
    out = []
    for t, n in enumerate(sizes):
        o = int(off_of[t])
        out.append(np.array(bufs[buf_of[t]][o:o + int(n)], copy=True))
    return out
