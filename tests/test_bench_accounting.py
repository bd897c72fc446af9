"""The benchmark's byte and flop accounting, pinned to the sizes written out
by hand (no GPU: only the arithmetic of bench.py is exercised)."""
import bench
import synth


def test_head_step_bytes_kd128():
    # S read + write 2*128*128*4, v 512, o 512, g + beta 8, q + k 2*128*4 / 3
    assert abs(bench.head_step_bytes(synth.DIMS128) - (131072 + 512 + 512 + 8 + 1024 / 3)) < 1e-9
    assert round(bench.head_step_bytes(synth.DIMS128), 2) == 132445.33


def test_head_step_bytes_kd64():
    assert abs(bench.head_step_bytes(synth.DIMS64) - (32768 + 256 + 256 + 8 + 512 / 3)) < 1e-9
    assert round(bench.head_step_bytes(synth.DIMS64), 2) == 33458.67


def test_m_step_bytes_share_one_state_pass():
    # M rows: the state is read and written once for all rows
    b8 = bench.head_step_bytes(synth.DIMS128, rows=8)
    assert abs(b8 - (131072 / 8 + 512 + 512 + 8 + 1024 / 3)) < 1e-9


def test_headline_launch_bytes():
    # 64 sequences x 48 layers x 48 value heads per launch
    hs = 64 * 48 * 48
    assert hs == 147456
    assert round(hs * bench.head_step_bytes(synth.DIMS128)) == 19529859072


def test_kernel_hash_sections_exist():
    for k in bench.HASH_SECTIONS:
        assert len(bench.kernel_hash(k)) == 16


def test_projection_shapes_reproduce_pages_weight_bytes():
    """The projection shapes read from the pages (one output per weight row)
    give the f32 weight bytes per layer and per token that the pages print."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "layer_weights_p24.json")))
    sh = gold["shape"]
    dims = (sh["vh"], sh["kh"], sh["kd"], sh["vd"])
    dim, vh, vd = sh["dim"], sh["vh"], sh["vd"]
    cd = synth.conv_dim_of(dims)
    floats = cd * dim + vh * vd * dim + 2 * vh * dim + dim * vh * vd
    per_layer = 4 * floats
    assert round(per_layer / 2**20) == gold["f32_weights_per_layer_MiB"]
    assert round(sh["layers"] * per_layer / 2**30) == gold["f32_weights_per_token_GiB"]
    # the benchmark's whole-layer weight bytes are the three large matrices
    assert synth.FE_DIM == dim and cd == 10240
    # the q4 layer: 4-bit weights with one binary16 scale per 32 for the three
    # large projections; in_proj_a / in_proj_b and the conv weights stay f32
    large = cd * dim + vh * vd * dim + dim * vh * vd
    q4 = large // 2 + (large // 32) * 2 + 4 * (2 * vh * dim + cd * 4)
    assert round(q4 / 2**20, 1) == gold["q4_weights_per_layer_MiB"]
    for block in (16, 64):                          # other block sizes miss the printed size
        other = large // 2 + (large // block) * 2 + 4 * (2 * vh * dim + cd * 4)
        assert round(other / 2**20, 1) != gold["q4_weights_per_layer_MiB"]


def test_frontend_bytes_written_out():
    # 128 rows of x (5120) and raw conv inputs (10240), Wa and Wb (48 x 5120
    # each), conv weights (10240 x 4 taps), the 3-frame history read and
    # written, and the q, k (16 x 128 each), v (48 x 128), g, beta outputs
    B, cd, dim = 128, 10240, 5120
    want = (B * dim + 2 * 48 * dim + B * cd + 2 * B * 3 * cd + cd * 4
            + B * (2 * 16 * 128 + 48 * 128 + 2 * 48)) * 4
    assert bench.frontend_bytes(B, synth.DIMS128) == want == 46743552
    # M rows share one history read; frontend_verify_m writes no history
    m8 = bench.frontend_bytes(B, synth.DIMS128, M=8, write_hist=False)
    assert m8 == (8 * B * dim + 2 * 48 * dim + 8 * B * cd + B * 3 * cd + cd * 4
                  + 8 * B * (2 * 16 * 128 + 48 * 128 + 2 * 48)) * 4


def test_m_step_variants_bytes():
    # verify_m reads the state once and writes none; a commit touches only
    # units with accepted rows (read + write) and reads their accepted rows
    tile = 128 * 128 * 4
    step_m = bench.head_step_bytes(synth.DIMS128, rows=8) * 8
    assert abs(step_m - (2 * tile + 8 * (512 + 512 + 8 + 1024 / 3))) < 1e-6
    row_no_o = bench.head_step_bytes(synth.DIMS128, write_o=False) - 2 * tile
    assert abs(row_no_o - (512 + 8 + 1024 / 3)) < 1e-9
