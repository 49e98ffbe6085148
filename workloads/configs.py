"""The five synthetic workloads.

The mask families are the ones the STOF pages list for the MHA experiments
(causal, sliding window, Longformer, BigBird, random/unstructured): STOF
explainer (gist.science) "Technical summary > Problem statement" and
"Experimental results > MHA performance"; the long-sequence length (16k)
follows "Experimental results > Scalability".  Shapes are model-shaped
(BERT-base, GPT-2/LLaMA, long context); no dataset or trained weights are
involved, the inputs are i.i.d. N(0,1) drawn from a fixed seed.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    cid: int          # also the seed of every random draw for this workload
    name: str
    B: int
    H: int
    S: int
    d: int
    dtype: str       # "f16" or "bf16": the Q/K/V element type
    family: str       # mask family, see workloads.gen.make_mask
    desc: str

    @property
    def n_ot(self):
        return -(-self.S // 64)


CONFIGS = {
    1: Config(1, "causal_s256", 1, 2, 256, 64, "f16", "causal",
              "causal j<=i, S=256"),
    2: Config(2, "bert_window_s512", 8, 12, 512, 64, "f16", "window64",
              "BERT-base shaped sliding window |i-j|<=64, S=512"),
    3: Config(3, "longformer_s2048", 4, 32, 2048, 128, "bf16", "longformer",
              "causal AND (|i-j|<=256 OR i<16 OR j<16), S=2048"),
    4: Config(4, "bigbird_s4096", 2, 16, 4096, 64, "f16", "bigbird",
              "64x64 blocks: 3 sliding + 2 global + 3 random per block row, "
              "20% of random-block elements dropped, S=4096"),
    5: Config(5, "long_unstructured_s16384", 1, 32, 16384, 128, "bf16",
              "long_random",
              "causal AND (|i-j|<=1024 OR Bernoulli(0.02)), S=16384"),
    # the row-wise kernel's regime (highly sparse): a measurement workload
    6: Config(6, "random_sparse_s4096", 1, 64, 4096, 64, "f16",
              "sparse_random", "Bernoulli(0.001) per element, S=4096"),
    # workload 5 without its band: the partial tiles a per-tile hybrid
    # would hand to a gather path, on their own (a measurement workload)
    7: Config(7, "far_random_s16384", 1, 32, 16384, 128, "bf16",
              "far_random", "causal AND Bernoulli(0.02), S=16384"),
}


def get_config(cid):
    return CONFIGS[int(cid)]
