"""gs_raster_fused_l1_noalloc (the fused forward + L1 + backward with its partial sums in
the library's static scratch array) against gs_raster_fused_l1 with a caller workspace,
through the C ABI: image, T_final, N_p, loss, the sum of N_p, the walk counts and the
per-Gaussian gradient sums bit for bit, on two calls in a row, the second on a smaller
scene and image.  GPU only.  Also: an image beyond the scratch's capacity is refused
before any launch."""
import pytest
import torch

from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import pipeline as PL
from differentiable_rasterization_amd import scenes
from tests.gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def _run(sc, noalloc):
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    c = B.camera_from(cam)
    params = PL.GaussianParams.from_scene(sc, DEV)
    st = PL.TrainStep(params, cam.width, cam.height, DEV, raster=rp)
    B.gs_project(params.gaussians(), c, rp, st.proj.abi())
    st.bins.sort(st.proj, c, rp)
    f = st.frame
    tgt = sc.targets[0].to(DEV)
    wc = torch.zeros(3, dtype=torch.int64, device=DEV)
    f.n_trav_sum.zero_()
    if noalloc:
        B.gs_raster_fused_l1_noalloc(params.gaussians(), st.bins.abi(), c, rp, tgt, f.color, f.t_final, f.n_trav,
                                     f.loss, f.n_trav_sum, walk_counts=wc)
    else:
        st.fused_l1(c, tgt, walk_counts=wc)
    B.gs_grad_aggregate(params.gaussians(), st.proj.abi(), st.bins.abi(), c, rp, st.grads2d, None)
    torch.cuda.synchronize()
    return [t.clone() for t in (f.color, f.t_final, f.n_trav, f.loss, f.n_trav_sum, wc, st.grads2d)]


@pytest.mark.parametrize("order", ["noalloc_first", "workspace_first"])
def test_fused_noalloc_matches_workspace_version(order):
    big = scenes.scene_100k()                       # 512 x 512
    small = scenes.scene_small_random(12, 3000, 130, 33, 2, extent=1.5, distance=3.0, log_scale_mean=-3.0)
    for sc in (big, small):                          # the second call is smaller
        log(f"no-alloc fused raster: {sc.name} {sc.cameras[0].width}x{sc.cameras[0].height} ({order})")
        runs = {}
        for noalloc in ((True, False) if order == "noalloc_first" else (False, True)):
            runs[noalloc] = _run(sc, noalloc)
        for a, b, nm in zip(runs[True], runs[False], ("color", "t_final", "n_trav", "loss", "n_trav_sum",
                                                      "walk_counts", "grads2d")):
            assert torch.equal(a, b), nm
        assert int(runs[True][4]) > 0 and float(runs[True][6].abs().max()) > 0.0


def test_fused_noalloc_refuses_images_beyond_its_scratch():
    sc = scenes.scene_small_random(12, 300, 64, 64, 1)
    rp = B.make_params(sc.sh_degree)
    params = PL.GaussianParams.from_scene(sc, DEV)
    cam = B.camera_from(sc.cameras[0])
    big = B.make_camera(list(cam.viewmat), cam.fx, cam.fy, cam.cx, cam.cy, 4096 + 16, 4096)
    bins = PL.Binning(sc.n, 64, 64, capacity=1024, device=DEV)
    img = torch.zeros(1, dtype=torch.float32, device=DEV)
    n = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(B.GsError) as e:
        B.gs_raster_fused_l1_noalloc(params.gaussians(), bins.abi(), big, rp, img, img, img, n, None, None)
    assert e.value.status == B.GS_ERR_UNSUPPORTED and "static scratch" in str(e.value)
