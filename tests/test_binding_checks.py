"""The binding rejects bad tensors before anything reaches the library: every
pointer argument must be a contiguous device tensor of the right dtype and
shape, on the same device as H.  The CPU tests run without a GPU; the GPU
tests check the remaining cases (a CPU tensor among device ones, a wrong
dtype or shape of an output) and that no kernel was launched."""
import pytest
import torch

import lm_head_top_amd as kd


def test_dev_tensor_rejects_host_dtype_shape_and_layout():
    x = torch.zeros(4, 3, dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        kd._dev_tensor(torch, x, "x", torch.float32, (4, 3))
    with pytest.raises(TypeError, match="must be torch.bfloat16"):
        kd._dev_tensor(torch, x, "x", torch.bfloat16, (4, 3))
    with pytest.raises(TypeError, match="torch.Tensor"):
        kd._dev_tensor(torch, [1.0], "x", torch.float32)


def test_entry_points_reject_host_tensors_before_loading_anything():
    H = torch.zeros(8, 16, dtype=torch.bfloat16)
    W = torch.zeros(32, 16, dtype=torch.bfloat16)
    idx = torch.zeros(8, 4, dtype=torch.int32)
    t = torch.zeros(8, 4, dtype=torch.float32)
    lse = torch.zeros(8, dtype=torch.float32)
    for call in (lambda: kd.forward(H, W, idx, t),
                 lambda: kd.backward(H, W, idx, t, lse),
                 lambda: kd.forward_ex(H, W, idx, t),
                 lambda: kd.backward_ex(H, W, idx, t, lse),
                 lambda: kd.forward_keep(H, W, idx, t),
                 lambda: kd.dense_forward(H, W, torch.zeros(8, 32)),
                 lambda: kd.dense_backward(H, W, torch.zeros(8, 32), lse, lse),
                 lambda: kd.topk_select(torch.zeros(8, 32), 4),
                 lambda: kd.validate(idx, 32)):
        with pytest.raises(ValueError, match="device tensor"):
            call()


def test_shape_and_rank_mismatches_are_rejected():
    H = torch.zeros(8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="2-D"):
        kd.forward(H, torch.zeros(32, dtype=torch.bfloat16), torch.zeros(8, 4, dtype=torch.int32),
                   torch.zeros(8, 4))


def _gpu_case(N=64, D=32, V=512, K=4):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    H = torch.randn(N, D, device=dev, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, D, device=dev, generator=g) / D ** 0.5).to(torch.bfloat16)
    idx = torch.randint(0, V, (N, K), device=dev, generator=g, dtype=torch.int32)
    t = torch.randn(N, K, device=dev, generator=g)
    return H, W, idx, t


def _no_launch(call, exc):
    """`call` raises `exc` and launches no kernel of the library."""
    names = tuple(kd.KERNELS)
    torch.cuda.synchronize()
    kd.profile_enable(names)
    for k in names:
        kd.profile_read(k)
    try:
        with pytest.raises(exc):
            call()
        torch.cuda.synchronize()
    finally:
        kd.profile_enable(None)
    assert sum(kd.profile_read(k)[1] for k in names) == 0


@pytest.mark.gpu
def test_backward_rejects_host_and_mis_typed_arguments():
    kd.load_library()
    H, W, idx, t = _gpu_case()
    N, D = H.shape
    V = W.shape[0]
    loss, lse = kd.forward(H, W, idx, t, 1.0, 32)
    torch.cuda.synchronize()
    dev = H.device
    _no_launch(lambda: kd.backward(H, W, idx, t, lse, torch.tensor([1.0]), 1.0, 32), ValueError)
    _no_launch(lambda: kd.backward(H, W, idx, t, lse.cpu(), None, 1.0, 32), ValueError)
    _no_launch(lambda: kd.backward(H, W, idx, t, lse, None, 1.0, 32,
                                   dW=torch.zeros(V, D, dtype=torch.bfloat16, device=dev)), TypeError)
    _no_launch(lambda: kd.backward(H, W, idx, t, lse, None, 1.0, 32,
                                   dW=torch.zeros(V - 1, D, device=dev)), ValueError)
    _no_launch(lambda: kd.backward(H, W, idx, t, lse, None, 1.0, 32,
                                   dW=torch.zeros(D, V, device=dev).t()), ValueError)
    _no_launch(lambda: kd.backward(H, W, idx, t, lse[:-1], None, 1.0, 32), ValueError)
    _no_launch(lambda: kd.backward(H, W, idx, t.cpu(), lse, None, 1.0, 32), ValueError)
    _no_launch(lambda: kd.backward(H, W, idx, t, lse, None, 1.0, 32,
                                   workspace=torch.empty(16, dtype=torch.uint8, device=dev)), ValueError)
    _no_launch(lambda: kd.backward_ex(H, W, idx, t, lse, None, 1.0, 32,
                                      row_weight=torch.ones(N)), ValueError)
    _no_launch(lambda: kd.backward_ex(H, W, idx, t, lse, None, 1.0, 32,
                                      labels=torch.zeros(N, dtype=torch.int64, device=dev)), TypeError)


@pytest.mark.gpu
def test_other_entry_points_reject_mis_typed_arguments():
    kd.load_library()
    H, W, idx, t = _gpu_case()
    N, D = H.shape
    V = W.shape[0]
    dev = H.device
    teacher = torch.randn(N, V, device=dev)
    loss, lse, lse_t = kd.dense_forward(H, W, teacher, 1.0, 32)
    torch.cuda.synchronize()
    _no_launch(lambda: kd.dense_backward(H, W, teacher, lse, lse_t, None, 1.0, 32,
                                         dW=torch.zeros(V, D, dtype=torch.bfloat16, device=dev)), TypeError)
    _no_launch(lambda: kd.dense_backward(H, W, teacher, lse, lse_t.cpu(), None, 1.0, 32), ValueError)
    _no_launch(lambda: kd.dense_backward(H, W, teacher, lse, lse_t, torch.tensor([1.0]), 1.0, 32),
               ValueError)
    _no_launch(lambda: kd.dense_forward(H, W, teacher[:, :-4], 1.0, 32), ValueError)
    _, _, ws = kd.forward_keep(H, W, idx, t, 1.0, 32)
    torch.cuda.synchronize()
    _no_launch(lambda: kd.backward_keep(H, W, idx.shape[1], ws, None, 1.0, 32,
                                        dW=torch.zeros(V, D, dtype=torch.float16, device=dev)), TypeError)
    _no_launch(lambda: kd.backward_keep(H, W, idx.shape[1], ws[:1024], None, 1.0, 32), ValueError)
    _no_launch(lambda: kd.backward_keep(H, W, idx.shape[1], ws.cpu(), None, 1.0, 32), ValueError)
    _no_launch(lambda: kd.topk_select(teacher.t(), 4), ValueError)
