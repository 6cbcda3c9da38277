"""The five workload configurations of the CSA / HCA hot path.

Hyper-parameters follow the DeepSeek-V4 digest (ai-papers-daily page
"DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence"),
模块 B configuration (m = 4, n_win = 128, head dim c = 512, 64 query heads,
d_c = 1024 for the Flash model) and 模块 C (m' = 128), scaled down where the
workload names smaller shapes.
"""

F32, BF16 = 0, 1
ROW_F32, ROW_BF16, ROW_FP8_ROPE_BF16, ROW_MXFP4 = 0, 1, 2, 3

CTX_1M = 1 << 20

CONFIGS = {
    1: dict(name="csa_fp32_n1024", kind="csa_prefill", seed=0, act=F32,
            n=1024, d=256, c=64, nh=8, m=4, cI=32, hI=4, k=16, n_win=64,
            kv_layout=ROW_F32, key_layout=ROW_F32, q_std=1.0),
    2: dict(name="hca_bf16_n32768", kind="hca_prefill", seed=1, act=BF16,
            n=32768, d=1024, c=128, nh=16, mp=128, n_win=128,
            kv_layout=ROW_BF16, q_std=1.0),
    3: dict(name="csa_prefill_bf16_n65536", kind="csa_prefill", seed=2, act=BF16,
            n=65536, d=2048, c=128, nh=64, m=4, cI=64, hI=32, k=512, n_win=128, d_c=512,
            kv_layout=ROW_BF16, key_layout=ROW_BF16, q_std=0.5),
    4: dict(name="csa_decode_b16_ctx1m", kind="csa_decode", seed=3, act=BF16,
            B=16, ctx=CTX_1M, c=512, nh=64, m=4, mp=128, cI=64, hI=32, k=1024, n_win=128,
            kv_layout=ROW_FP8_ROPE_BF16, key_layout=ROW_MXFP4, q_std=1.0),
    5: dict(name="csa_hca_pair_chunk8192_ctx1m", kind="pair", seed=4, act=BF16,
            n=8192, n_left=4, ctx=CTX_1M, d=4096, c=512, nh=64, m=4, mp=128, cI=64, hI=32,
            k=1024, n_win=128, d_c=1024,
            kv_layout=ROW_FP8_ROPE_BF16, key_layout=ROW_MXFP4, q_std=0.5),
}


def config(i):
    return dict(CONFIGS[i])
