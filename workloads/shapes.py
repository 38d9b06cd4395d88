"""Flat parameter-arena layouts of the models the pages train.

The arena is one flat buffer per replica ("Distributed training" (noeira),
"Four strategies, one interface": one flat buffer for the weights, one for
the gradients).  Tensors sit in forward order: embeddings, then each block,
then the final norm (and, for Llama, the untied output head).  ``layer`` is -1
for the embeddings, 0..L-1 for the blocks and L for what follows them.

Sizes (each reproduces the parameter count quoted for the model):

* char GPT 6 x 384, 6 heads, vocabulary 65, context 256: 10,770,816
  (20 bytes per parameter is the 215.4 MB of DDP state per GPU that
  "Distributed training" reports for it at N = 8).
* GPT-2 124M (12 x 768, vocabulary 50257, context 1024): 124,439,808.
* GPT-2 1.5B (48 x 1600): 1,557,611,200.
* Llama-shaped 7B (32 x 4096, FFN 11008, vocabulary 32000, untied head):
  6,738,415,616.
"""

from dataclasses import dataclass, field


@dataclass
class Arena:
    name: str
    tensors: list = field(default_factory=list)  # (name, numel, layer)

    @property
    def numel(self):
        return sum(n for _, n, _ in self.tensors)

    @property
    def numels(self):
        return [n for _, n, _ in self.tensors]

    def spans(self):
        """(offset, numel, layer) of every tensor, in arena order."""
        out, pos = [], 0
        for _, n, layer in self.tensors:
            out.append((pos, n, layer))
            pos += n
        return out


def gpt2(n_layer, d, vocab, ctx, name="gpt2"):
    t = [("wte", vocab * d, -1), ("wpe", ctx * d, -1)]
    for l in range(n_layer):
        t += [
            (f"h{l}.ln1.w", d, l), (f"h{l}.ln1.b", d, l),
            (f"h{l}.qkv.w", d * 3 * d, l), (f"h{l}.qkv.b", 3 * d, l),
            (f"h{l}.proj.w", d * d, l), (f"h{l}.proj.b", d, l),
            (f"h{l}.ln2.w", d, l), (f"h{l}.ln2.b", d, l),
            (f"h{l}.fc.w", d * 4 * d, l), (f"h{l}.fc.b", 4 * d, l),
            (f"h{l}.fcproj.w", 4 * d * d, l), (f"h{l}.fcproj.b", d, l),
        ]
    t += [("lnf.w", d, n_layer), ("lnf.b", d, n_layer)]
    return Arena(name, t)


def char_gpt():
    return gpt2(6, 384, 65, 256, name="char_gpt_6x384")


def llama(n_layer, d, ffn, vocab, name="llama"):
    t = [("embed", vocab * d, -1)]
    for l in range(n_layer):
        t += [
            (f"l{l}.attn_norm", d, l),
            (f"l{l}.q", d * d, l), (f"l{l}.k", d * d, l),
            (f"l{l}.v", d * d, l), (f"l{l}.o", d * d, l),
            (f"l{l}.ffn_norm", d, l),
            (f"l{l}.gate", d * ffn, l), (f"l{l}.up", d * ffn, l),
            (f"l{l}.down", ffn * d, l),
        ]
    t += [("norm", d, n_layer), ("lm_head", vocab * d, n_layer)]
    return Arena(name, t)


def flat(numel, name):
    return Arena(name, [("flat", numel, 0)])


ARENAS = {
    "tiny": lambda: flat(4096, "tiny_4096"),
    "char_gpt": char_gpt,
    "gpt2_124m": lambda: gpt2(12, 768, 50257, 1024, name="gpt2_124m"),
    "gpt2_1p5b": lambda: gpt2(48, 1600, 50257, 1024, name="gpt2_1p5b"),
    "llama_7b": lambda: llama(32, 4096, 11008, 32000, name="llama_7b"),
}


def arena(name):
    return ARENAS[name]()
