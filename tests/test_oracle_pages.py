"""The oracle's constants against the numbers the Hy-Nomas pages print
(tests/golden/page_constants.json, each entry cited)."""
import json
import os

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def val(k):
    return GOLD[k]["value"]


def test_head_geometry():
    assert val("heads") * val("head_dim") == val("hidden")
    assert oracle.D == val("head_dim")
    assert sum(val("rope_axes")) == val("head_dim")
    assert tuple(oracle.AXES) == tuple(val("rope_axes"))
    assert oracle.THETA == val("rope_theta")
    assert list(oracle.AXIS_OFFSETS) == [0, 16, 72]


def test_tokens_per_latent_frame():
    w, h = val("frame_px")
    s = val("vae_spatial")
    assert val("patch") == [1, 1, 1]
    assert (w // s, h // s) == (40, 22)
    assert (w // s) * (h // s) == 880
    assert synth.HG * synth.WG == 880 and (synth.HG, synth.WG) == (h // s, w // s)


def test_latent_frames_per_second():
    # 240 video frames -> [30, 30] latent frames (4x temporal compression)
    gold = GOLD["diffusers_segment_latents"]
    assert gold["num_frames"] // val("vae_temporal") == sum(gold["value"])
    assert val("fps") // val("vae_temporal") == 6
    # a 12 s turn is 72 latent frames = 288 video frames = 72 camera tokens
    assert 12 * val("fps") // val("vae_temporal") == 72
    assert synth.turn_seg(0).T == 72 and synth.WORKLOADS["fiveturns"].cam_frames == 12 * val("fps")


def test_camera_token_width():
    assert val("cam_group_frames") * 16 == val("cam_token_dim")


def test_history_window_in_workloads():
    for name in ("turn3s", "seg4s"):
        (hseg,) = synth.WORKLOADS[name].hist_segs
        assert hseg.T == val("history_latent_frames")
